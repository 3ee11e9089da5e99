// libgpt2mi: C ABI of the fp32 GPT-2 training step on gfx950 (include/gpt2.h,
// include/gpt2_kernels.h).  Host side: buffer layout, argument checks, and the
// ordered launch sequence of forward, backward and AdamW on one HIP stream.
//
// The sequence follows the block dataflow of the GeekNews page on the
// 3000-byte C GPT-2 ("Phần lõi Transformer"): LayerNorm -> qkv linear ->
// causal attention -> projection + residual -> LayerNorm -> fc linear ->
// GELU -> projection + residual, then the final LayerNorm and the product
// with the token-embedding weights; and the QbitAI/InfoQ llm.c articles'
// scheme of one allocation made up front with every tensor at a fixed offset
// and a hand-written backward per layer.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <queue>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/gpt2.h"
#include "../../include/gpt2_kernels.h"
#include "../../include/gpt2_audit.h"
#include "attention.h"
#include "audit.h"
#include "checkpoint.h"
#include "common.h"
#include "decode.h"
#include "gemm.h"
#include "probe.h"
#include "kernels.h"
#include "status.h"

namespace {

thread_local std::string g_last_error;

constexpr size_t ALIGN = 64;  // floats: every tensor offset is a multiple of 256 bytes
inline size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

const char *kParamNames[16] = {"wte",  "wpe",  "ln1w", "ln1b", "qkvw", "qkvb",    "attprojw", "attprojb",
                               "ln2w", "ln2b", "fcw",  "fcb",  "fcprojw", "fcprojb", "lnfw",  "lnfb"};

enum ActId {
    A_ENCODED, A_LN1, A_LN1_MEAN, A_LN1_RSTD, A_QKV, A_ATT, A_ATTY, A_RES2, A_LN2, A_LN2_MEAN, A_LN2_RSTD,
    A_FCH, A_FCH_GELU, A_RES3, A_LNF, A_LNF_MEAN, A_LNF_RSTD, A_LOGITS, A_LOSSES, A_LOSS, A_LSE, NUM_ACTS
};
const char *kActNames[NUM_ACTS] = {"encoded", "ln1",      "ln1_mean", "ln1_rstd",  "qkv",      "att",
                                   "atty",    "residual2", "ln2",     "ln2_mean",  "ln2_rstd", "fch",
                                   "fch_gelu", "residual3", "lnf",    "lnf_mean",  "lnf_rstd", "logits",
                                   "losses",  "loss",     "lse"};

// How a GEMM is launched: tile shape and number of K splits.
struct Plan {
    int tile;
    int ksplit;
};

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// Launch planning.  Work is spread over 256 CUs; a CU holds up to `occ`
// workgroups of a tile shape at once (register/LDS limited) and reaches full
// MFMA throughput with two or more resident.  Workgroups are all the same
// size, so a CU with n of them runs rounds of min(occ, left) at a time, and
// a round of k costs max(k, 2) tile-times.  The plan with the least
// predicted time wins; a split of K adds the traffic of writing and summing
// the partial products.  The per-shape efficiencies are measured values of
// the kernel on long runs at this occupancy.
struct TileShape {
    int bm, bn, occ;
    double eff;
};
const TileShape kTiles[5] = {
    {0, 0, 0, 0.0}, {128, 128, 3, 0.73}, {128, 64, 4, 0.68}, {64, 64, 6, 0.66}, {64, 192, 3, 0.70}};

// A product whose tiles do not all fit inside it (or whose K is not a whole
// number of 32-wide slices) runs the kernel with bounds tests in its K loop,
// measured at about 0.8 of the whole-tile kernel's rate (GPT-2 XL, C = 1600:
// 57 to 65 % of the matrix peak against 72 to 76 % for whole tiles).
constexpr double kPartialTileEff = 0.8;
bool tiles_whole(int M, int N, int K, int tile) {
    return M % kTiles[tile].bm == 0 && N % kTiles[tile].bn == 0 && K % 32 == 0;
}
double tile_eff(int M, int N, int K, int tile) {
    return kTiles[tile].eff * (tiles_whole(M, N, K, tile) ? 1.0 : kPartialTileEff);
}

double predict_gemm_us(int M, int N, int K, long long batches, int tile, int ks) {
    const TileShape &t = kTiles[tile];
    const double eff = tile_eff(M, N, K, tile);
    const long long wgs = ceil_div(M, t.bm) * ceil_div(N, t.bn) * batches * ks;
    // equal workgroups run in rounds of up to occ per CU: the CU with the
    // most sets the time, a round of k costing max(k, 2) tile-times (a short
    // last round costs nearly a full one)
    double units = 0;
    long long n = ceil_div(wgs, 256);
    while (n > 0) {
        long long k = n < t.occ ? n : t.occ;
        units += k > 2 ? k : 2;
        n -= k;
    }
    const double kc = (double)ceil_div(ceil_div(K, ks), 32) * 32;
    const double cu_flops_per_us = 157.3e6 / 256.0;
    double us = units * (2.0 * t.bm * t.bn * kc) / (eff * cu_flops_per_us);
    if (ks > 1) us += 8.0 + (2.0 * ks + 2.0) * M * N * 4.0 / 5.0e6;  // extra launch + partials written, read, summed
    return us;
}

Plan plan_gemm(int M, int N, int K, long long batches, bool allow_split) {
    Plan best{1, 1};
    double best_us = 1e30;
    static const int splits[] = {1, 2, 3, 4, 6, 8, 12, 16};
    for (int tile = 1; tile <= 4; tile++) {
        if (N <= 64 && (tile == 1 || tile == 4)) continue;
        for (int ks : splits) {
            if (ks > 1 && (!allow_split || K / ks < 256)) break;
            double us = predict_gemm_us(M, N, K, batches, tile, ks);
            if (us < best_us * 0.98) {
                best_us = us;
                best = Plan{tile, ks};
            }
        }
    }
    return best;
}

// Planning of a weight gradient and an input gradient launched as one grid
// (gemm_launch_pair).  Workgroups of unequal length share the CUs, so the
// time is simulated: workgroups are dealt to the 256 CUs in grid order, a
// CU holds up to `occ` of them and shares its rate among those resident
// (full rate from two up, half rate with one), and a freed slot takes the
// next workgroup.  Each workgroup's work is its tile's flops at the tile
// shape's measured efficiency plus a fixed cost.
struct WgGroup {
    long long count;
    double us;  // one workgroup alone on a CU at full rate
};
// fixed cost of a workgroup (first operand loads, epilogue), fitted to
// measured pair timings at the GPT-2 layer shapes
const double kWgFixedUs = 2.0;

double simulate_us(int occ, const std::vector<WgGroup> &groups) {
    const int NCU = 256;
    struct Cu {
        double t = 0;            // time of the last update
        std::vector<double> rem;  // remaining work of the resident workgroups
        int ver = 0;
    };
    std::vector<Cu> cu(NCU);
    size_t gi = 0;
    long long left = groups.empty() ? 0 : groups[0].count;
    auto next_wg = [&](double &w) {
        while (gi < groups.size() && left == 0) {
            if (++gi < groups.size()) left = groups[gi].count;
        }
        if (gi >= groups.size()) return false;
        left--;
        w = groups[gi].us;
        return true;
    };
    auto speed = [](size_t k) { return k >= 2 ? 1.0 / (double)k : 0.5; };
    typedef std::tuple<double, int, int> Ev;  // completion time, cu, version
    std::priority_queue<Ev, std::vector<Ev>, std::greater<Ev>> pq;
    auto schedule = [&](int c) {
        Cu &u = cu[c];
        u.ver++;
        if (u.rem.empty()) return;
        double mn = u.rem[0];
        for (double r : u.rem) mn = r < mn ? r : mn;
        pq.push(Ev(u.t + mn / speed(u.rem.size()), c, u.ver));
    };
    double w;
    for (int k = 0; k < occ; k++)
        for (int c = 0; c < NCU; c++)
            if (next_wg(w)) cu[c].rem.push_back(w);
    for (int c = 0; c < NCU; c++) schedule(c);
    double end = 0;
    while (!pq.empty()) {
        Ev ev = pq.top();
        pq.pop();
        const double t = std::get<0>(ev);
        const int c = std::get<1>(ev);
        Cu &u = cu[c];
        if (std::get<2>(ev) != u.ver) continue;
        const double done = (t - u.t) * speed(u.rem.size());
        std::vector<double> keep;
        for (double r : u.rem)
            if (r - done > 1e-9) keep.push_back(r - done);
        u.rem.swap(keep);
        u.t = t;
        end = t > end ? t : end;
        while ((int)u.rem.size() < occ && next_wg(w)) u.rem.push_back(w);
        schedule(c);
    }
    return end;
}

double split_overhead_us(int ks, long long M, long long N) {
    return ks > 1 ? 8.0 + (2.0 * ks + 2.0) * M * N * 4.0 / 5.0e6 : 0.0;
}

struct PairPlan {
    bool pair;
    int tile, ks_dw, ks_dinp;
};

// dW[OC][K] += dout^T inp (reduction over N) beside dinp[N][K] = dout W
// (reduction over OC); the input gradient may split K only if allowed.  The
// pair always runs as one grid: measured, that beats two launches (whose
// ramp-up and drain the model does not see); the model picks the tile shape
// and the splits.
PairPlan plan_pair(int N, int K, int OC, bool split_dinp) {
    static std::mutex mu;
    static std::map<std::tuple<int, int, int, bool>, PairPlan> cache;
    std::lock_guard<std::mutex> lock(mu);
    auto key = std::make_tuple(N, K, OC, split_dinp);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    // Plans that measured faster on MI355X than the model's choice (whole-step
    // timings with per-launch events, the model's plan beside the hint), at the
    // exact shapes they were measured at: the MLP output projection of GPT-2
    // 124M at B = 4 and 16, where 128 x 64 tiles (four workgroups per CU)
    // beat the 128 x 128 tiles the model prefers (3.52 against 4.05 ms per
    // step at B = 4, 13.60 against 13.91 at B = 16); the MLP input
    // projection of GPT-2 XL, where 64 x 64 tiles (4100 workgroups, six per
    // CU) beat the model's 128 x 64 (63.2 against 73.9 ms per step); at
    // 124M B = 16, 128 x 64 tiles with four K splits of the weight gradient
    // for the MLP input and QKV projections and 64 x 64 tiles for the
    // attention projection (14.63 against 15.47, 10.98 against 11.09 on a
    // box 3 % slower, 3.74 against 3.83 ms per step).  At the
    // 124M B = 4 layer shapes the model's plans stayed faster than the
    // alternatives tried (64 x 64 for fc: 3.83 against 3.72 ms; 128 x 64
    // for qkv: 3.12 against 2.93; 64 x 64 for attproj: 1.06 against 1.02).
    struct Hint {
        int N, K, OC;
        bool split_dinp;
        PairPlan plan;
    };
    static const Hint kHints[] = {{4096, 3072, 768, false, {true, 2, 2, 1}},
                                  {16384, 3072, 768, false, {true, 2, 2, 1}},
                                  {4096, 1600, 6400, false, {true, 3, 1, 1}},
                                  {16384, 768, 3072, false, {true, 2, 4, 1}},
                                  {16384, 768, 768, false, {true, 3, 4, 1}},
                                  {16384, 768, 2304, false, {true, 2, 4, 1}}};
    for (const Hint &h : kHints)
        if (h.N == N && h.K == K && h.OC == OC && h.split_dinp == split_dinp) return cache[key] = h.plan;
    double best = 1e30;
    PairPlan bp{true, 1, 1, 1};
    static const int splits[] = {1, 2, 3, 4, 6, 8, 12, 16};
    const double cu_flops_per_us = 157.3e6 / 256.0;
    for (int tile = 1; tile <= 3; tile++) {
        const TileShape &t = kTiles[tile];
        if (K <= 64 && tile == 1) continue;
        // the paired kernel runs without bounds tests only when both products are whole
        const bool whole = tiles_whole(OC, K, N, tile) && tiles_whole(N, K, OC, tile);
        const double eff = t.eff * (whole ? 1.0 : kPartialTileEff);
        for (int kd : splits) {
            if (kd > 1 && N / kd < 256) break;
            for (int ki : splits) {
                if (ki > 1 && (!split_dinp || OC / ki < 256)) break;
                const double kcd = (double)ceil_div(ceil_div(N, kd), 32) * 32;
                const double kci = (double)ceil_div(ceil_div(OC, ki), 32) * 32;
                std::vector<WgGroup> g = {
                    {ceil_div(OC, t.bm) * ceil_div(K, t.bn) * kd, kWgFixedUs + 2.0 * t.bm * t.bn * kcd / (eff * cu_flops_per_us)},
                    {ceil_div(N, t.bm) * ceil_div(K, t.bn) * ki, kWgFixedUs + 2.0 * t.bm * t.bn * kci / (eff * cu_flops_per_us)}};
                const double us = simulate_us(t.occ, g) + split_overhead_us(kd, OC, K) + split_overhead_us(ki, N, K);
                if (us < best * 0.98) {
                    best = us;
                    bp = PairPlan{true, tile, kd, ki};
                }
            }
        }
    }
    cache[key] = bp;
    return bp;
}

// Floats of split-K partials a linear layer's backward may need, for the
// input gradient and the weight gradient (as separate launches or as a pair).
void bwd_split_need(int N, int K, int OC, bool split_dinp, size_t &sk_dinp, size_t &sk_dw) {
    const Plan sd = plan_gemm(OC, K, N, 1, true), si = plan_gemm(N, K, OC, 1, split_dinp);
    const PairPlan pp = plan_pair(N, K, OC, split_dinp);
    size_t a = si.ksplit > 1 ? (size_t)si.ksplit * N * K : 0, b = sd.ksplit > 1 ? (size_t)sd.ksplit * OC * K : 0;
    if (pp.pair && pp.ks_dinp > 1) a = std::max(a, (size_t)pp.ks_dinp * N * K);
    if (pp.pair && pp.ks_dw > 1) b = std::max(b, (size_t)pp.ks_dw * OC * K);
    sk_dinp = std::max(sk_dinp, a);
    sk_dw = std::max(sk_dw, b);
}

// The K split linear_bwd uses for the weight gradient (with an input gradient
// beside it, whose own split is allowed or not).
int dw_ksplit(int N, int K, int OC, bool split_dinp) {
    const PairPlan pp = plan_pair(N, K, OC, split_dinp);
    return pp.pair ? pp.ks_dw : plan_gemm(OC, K, N, 1, true).ksplit;
}

// The four weight-gradient sites of a layer: (in, out) features and the
// parameter tensors of the weight and the bias.
enum { SITE_QKV = 0, SITE_ATTPROJ = 1, SITE_FC = 2, SITE_FCPROJ = 3, NSITES = 4 };

struct Layout {
    int B, T, C, L, NH, V, Vp, maxT, hd;
    bool flash;  // fused attention (no T x T matrices kept)
    long long BT;
    size_t poff[16], pcnt[16], nparams;
    size_t aoff[NUM_ACTS], acnt[NUM_ACTS], nacts;
    // work buffer
    size_t w_dres, w_dln, w_datty, w_dqkv, w_dfch, w_datt, w_flash, w_part, w_splitk, w_splitk_dw, w_dbias, w_dec,
        nwork;
    // per-layer split-K partials of each site's weight / bias gradient, summed
    // for all layers at the end of the backward (ks 1: none)
    int site_ks[NSITES];
    size_t w_site_dw[NSITES], w_site_db[NSITES];
    // int buffer
    size_t i_tok, i_order, i_sort, i_err, i_dec, niwork;
    // the work regions with their exact float counts (offsets are padded to
    // 64 floats), each cut into `parts` equal slices (per layer or per slot)
    struct WRegion {
        const char *name;
        size_t off, cnt;
        int parts;
    };
    WRegion wreg[24];
    int nwreg;
};

bool config_ok(const gpt2_config *c, int B, int T, std::string *why) {
    char buf[256];
    auto fail = [&](const char *m) {
        if (why) *why = m;
        return false;
    };
    if (!c) return fail("config is NULL");
    if (c->max_seq_len <= 0 || c->vocab_size <= 0 || c->num_layers <= 0 || c->num_heads <= 0 || c->channels <= 0)
        return fail("config fields must be positive");
    if (c->padded_vocab_size < c->vocab_size) return fail("padded_vocab_size < vocab_size");
    if (c->padded_vocab_size % 4) return fail("padded_vocab_size must be a multiple of 4");
    if (c->channels % c->num_heads) return fail("channels must be a multiple of num_heads");
    if (c->channels % 4 || (c->channels / c->num_heads) % 4)
        return fail("channels and head dimension must be multiples of 4");
    if (c->channels > 2048) return fail("channels > 2048 is not supported");
    if (B <= 0 || T <= 0) return fail("B and T must be positive");
    if (T > c->max_seq_len) return fail("T > max_seq_len");
    if (T > 1024) return fail("T > 1024 is not supported");
    // the materialised attention (head dims without the fused kernels) keeps
    // T x T matrices read 16 bytes at a time along T
    if (T % 4 && !flash_attention_supported(c->channels / c->num_heads))
        return fail("T must be a multiple of 4 for head dims other than 16, 32 and 64");
    if ((long long)B * T > (1LL << 24)) return fail("B*T too large");
    snprintf(buf, sizeof buf, "ok");
    return true;
}

void make_layout(const gpt2_config *c, int B, int T, Layout *Lo) {
    Layout &l = *Lo;
    l.B = B; l.T = T; l.C = c->channels; l.L = c->num_layers; l.NH = c->num_heads; l.V = c->vocab_size;
    l.Vp = c->padded_vocab_size; l.maxT = c->max_seq_len; l.hd = l.C / l.NH;
    l.BT = (long long)B * T;
    const size_t C = l.C, L = l.L, BT = l.BT, NH = l.NH, TT = (size_t)T * T;
    size_t n[16] = {(size_t)l.Vp * C, (size_t)l.maxT * C, L * C, L * C, L * 3 * C * C, L * 3 * C, L * C * C, L * C,
                    L * C, L * C, L * 4 * C * C, L * 4 * C, L * C * 4 * C, L * C, C, C};
    size_t off = 0;
    for (int i = 0; i < 16; i++) {
        l.poff[i] = off;
        l.pcnt[i] = n[i];
        off += n[i];
    }
    l.nparams = off;
    l.flash = flash_attention_supported(l.hd);
    const size_t natt = l.flash ? 0 : L * B * NH * TT, nlse = l.flash ? L * B * NH * (size_t)T : 0;
    size_t a[NUM_ACTS] = {BT * C,      L * BT * C,  L * BT,     L * BT,     L * BT * 3 * C, natt,
                          L * BT * C,  L * BT * C,  L * BT * C, L * BT,     L * BT,         L * BT * 4 * C,
                          L * BT * 4 * C, L * BT * C, BT * C,   BT,         BT,             BT * (size_t)l.Vp,
                          BT,          1,           nlse};
    off = 0;
    for (int i = 0; i < NUM_ACTS; i++) {
        l.aoff[i] = off;
        l.acnt[i] = a[i];
        off = align_up(off + a[i]);
    }
    l.nacts = off;

    off = 0;
    l.nwreg = 0;
    auto add_w = [&](const char *name, size_t cnt, int parts) {
        l.wreg[l.nwreg++] = Layout::WRegion{name, off, cnt, parts};
        const size_t at = off;
        off = align_up(off + cnt);
        return at;
    };
    l.w_dres = add_w("dres", BT * C, 1);
    l.w_dln = add_w("dln", BT * C, 1);
    l.w_datty = add_w("datty", BT * C, 1);
    l.w_dqkv = add_w("dqkv", BT * 3 * C, 1);
    l.w_dfch = add_w("dfch", BT * 4 * C, 1);
    l.w_datt = add_w("datt", l.flash ? (size_t)B * NH * T : (size_t)B * NH * TT, 1);
    l.w_flash = add_w("flash_ws", l.flash ? flash_attention_work(B, T, (int)C, (int)NH) : 0, 1);
    // LayerNorm parameter partials of all 2L + 1 LayerNorms (summed once at the end)
    l.w_part = add_w("ln_partials", (2 * L + 1) * (size_t)ln_partials((int)BT) * 2 * C, (int)(2 * L + 1));
    // split-K partial products: of the input gradient dlnf (the only one
    // allowed to split) and of the weight gradients, in separate regions
    // because a pair of them runs as one grid
    size_t sk = 0, sk_dw = 0;
    bwd_split_need((int)BT, (int)C, (int)(3 * C), false, sk, sk_dw);
    bwd_split_need((int)BT, (int)C, (int)C, false, sk, sk_dw);
    bwd_split_need((int)BT, (int)C, (int)(4 * C), false, sk, sk_dw);
    bwd_split_need((int)BT, (int)(4 * C), (int)C, false, sk, sk_dw);
    bwd_split_need((int)BT, (int)C, l.Vp, true, sk, sk_dw);
    l.w_splitk = add_w("splitk", sk, 1);
    l.w_splitk_dw = add_w("splitk_dw", sk_dw, 1);
    {
        static const char *dw_names[NSITES] = {"site_dw_qkv", "site_dw_attproj", "site_dw_fc", "site_dw_fcproj"};
        static const char *db_names[NSITES] = {"site_db_qkv", "site_db_attproj", "site_db_fc", "site_db_fcproj"};
        const int sin[NSITES] = {(int)C, (int)C, (int)C, (int)(4 * C)};
        const int sout[NSITES] = {(int)(3 * C), (int)C, (int)(4 * C), (int)C};
        for (int j = 0; j < NSITES; j++) {
            const int ks = dw_ksplit((int)BT, sin[j], sout[j], false);
            l.site_ks[j] = ks;
            const size_t kk = ks > 1 ? (size_t)ks : 0;
            l.w_site_dw[j] = add_w(dw_names[j], L * kk * sout[j] * sin[j], (int)L);
            l.w_site_db[j] = add_w(db_names[j], L * kk * sout[j], (int)L);
        }
    }
    l.w_dbias = add_w("dbias_ws", 16 * 4 * C, 1);
    // one decoding step's rows: residual x and attention output [B][C] each,
    // MLP hidden [B][4C], then the attention's per-chunk partials
    l.w_dec = add_w("decode", (size_t)B * 6 * C + decode_attention_work(B, T, (int)C, (int)NH), 1);
    l.nwork = off;
    l.i_tok = 0;
    l.i_order = align_up(BT);
    l.i_sort = l.i_order + align_up(BT);  // the token order's sorted chunks (8-byte keys), at large BT
    l.i_err = l.i_sort + align_up(k_token_prep_work((int)BT));
    l.i_dec = l.i_err + ALIGN;  // the position a decoding step works on (read on the device)
    l.niwork = l.i_dec + ALIGN;
}

// When a model's profiler is on, each launch of the step is bracketed by two
// HIP events on the model's stream and tagged with the kernel's name and its
// algorithmic FLOPs and bytes (compulsory operand traffic).
struct ProfRec {
    const char *name, *site;
    double flops, bytes;
    hipEvent_t a, b;
};
struct Profiler {
    bool on = false;
    hipStream_t stream = nullptr;
    std::vector<hipEvent_t> pool;
    size_t used = 0;
    std::vector<ProfRec> recs;
};

}  // namespace

struct gpt2_model {
    Layout lo;
    gpt2_buffers buf;
    hipStream_t stream;
    int mm_prec = GPT2_FP32;  // precision of the linear-layer products
    bool have_targets = false;
    // captured decoding steps, one per (tokens, coins, next) of the caller
    struct DecodeGraph {
        const int32_t *tokens;
        const float *coins;
        int32_t *next;
        hipGraphExec_t exec;
    };
    std::vector<DecodeGraph> decode_graphs;
    hipStream_t capture_stream = nullptr;
    bool graphs_ok = true;
    std::string err;
    Profiler prof;
};

namespace {

gpt2_status fail(gpt2_model *m, gpt2_status st, const std::string &msg) {
    if (m) m->err = msg;
    g_last_error = msg;
    return st;
}

}  // namespace

void set_last_error(const std::string &msg) { g_last_error = msg; }

namespace {

#define HIPCK(model, expr)                                                                             \
    do {                                                                                               \
        hipError_t e_ = (expr);                                                                        \
        if (e_ != hipSuccess)                                                                          \
            return fail(model, GPT2_EDEVICE, std::string(#expr) + ": " + hipGetErrorString(e_));      \
    } while (0)

#define KRUN(model, name, bytes, call) HIPCK(model, timed(name, 0.0, (double)(bytes), [&]() { return call; }))
#define KRUNF(model, name, flops, bytes, call) \
    HIPCK(model, timed(name, (double)(flops), (double)(bytes), [&]() { return call; }))

// ---------------------------------------------------------------- per-launch timing

thread_local Profiler *g_prof = nullptr;

thread_local const char *g_site = "";  // call site of the launches being made

template <class F>
hipError_t timed(const char *name, double flops, double bytes, F &&f) {
    Profiler *p = g_prof;
    if (!p) return f();
    while (p->used + 2 > p->pool.size()) {
        hipEvent_t e;
        hipError_t er = hipEventCreate(&e);
        if (er != hipSuccess) return er;
        p->pool.push_back(e);
    }
    hipEvent_t a = p->pool[p->used++], b = p->pool[p->used++];
    hipError_t e = hipEventRecord(a, p->stream);
    if (e != hipSuccess) return e;
    e = f();
    if (e != hipSuccess) return e;
    e = hipEventRecord(b, p->stream);
    p->recs.push_back({name, g_site, flops, bytes, a, b});
    return e;
}

// Names the call site of the launches made in its scope (profile entries are
// reported as "kernel|site").
struct Site {
    const char *saved;
    explicit Site(const char *s) : saved(g_site) { g_site = s; }
    ~Site() { g_site = saved; }
};

// Precision of the linear-layer products being launched (GPT2_FP32 or
// GPT2_BF16); attention products are always fp32.
thread_local int g_prec = GPT2_FP32;
struct PrecScope {
    int saved;
    explicit PrecScope(int prec) : saved(g_prec) { g_prec = prec; }
    ~PrecScope() { g_prec = saved; }
};

// Makes a model's profiler the active one for the duration of an API call.
struct ProfScope {
    Profiler *saved;
    explicit ProfScope(gpt2_model *m) : saved(g_prof) { g_prof = m && m->prof.on ? &m->prof : nullptr; }
    ~ProfScope() { g_prof = saved; }
};

// "kernel<hd>" as a kernel-trace profiler shows the fused attention kernels
// (static strings: profile records keep the pointer).
enum { FL_FWD = 0, FL_DKDV = 1 };
const char *flash_name(int which, int hd) {
    static const char *names[2][3] = {
        {"flash_fwd_kernel<16>", "flash_fwd_kernel<32>", "flash_fwd_kernel<64>"},
        {"flash_bwd_dkdv_kernel<16>", "flash_bwd_dkdv_kernel<32>", "flash_bwd_dkdv_kernel<64>"}};
    return names[which][hd == 16 ? 0 : (hd == 32 ? 1 : 2)];
}

// Every GEMM of the step goes through here (`site` overrides the caller's).
hipError_t gemm_run(const GemmDesc &d, hipStream_t s, const char *site = nullptr) {
    Site site_(site ? site : g_site);
    const double nb = (double)d.nbo * d.nbi;
    double flops, bytes;
    if (d.causal != CAUSAL_NONE) {
        // only the lower triangle (u <= t) of each T x T score matrix is work
        const double tri = 0.5 * d.M * (d.M + 1.0);
        const double inner = d.causal == CAUSAL_SKIP_UPPER ? d.K : d.N;
        flops = 2.0 * tri * inner * nb;
        bytes = 4.0 * nb * (tri + 2.0 * d.M * inner);
    } else {
        flops = 2.0 * d.M * d.N * d.K * nb;
        double out = (double)d.M * d.N * (d.ksplit > 1 ? d.ksplit : 1);
        if (d.epi == EPI_ACCUM || d.epi == EPI_RESID || d.epi == EPI_GELU || d.epi == EPI_GELU_BWD) out *= 2;
        bytes = 4.0 * nb * ((double)d.M * d.K + (double)d.K * d.N + out);
    }
    return timed(gemm_kernel_name(d), flops, bytes, [&]() { return gemm_launch(d, s); });
}

// ---------------------------------------------------------------- building blocks

// Device-to-device copy of n ids (declared, not made, during a launch audit).
hipError_t copy_ids(int32_t *dst, const int32_t *src, int n, hipStream_t s) {
    if (AuditSink *au = audit_sink()) {
        audit(au, "copy_ids", "src", src, n, false);
        audit(au, "copy_ids", "dst", dst, n, true);
        return hipSuccess;
    }
    return hipMemcpyAsync(dst, src, sizeof(int32_t) * n, hipMemcpyDeviceToDevice, s);
}

// Tile shape of a forward product: the model's choice, except at shapes
// where another measured faster on MI355X (whole-step timings with
// per-launch events, the model's plan beside the hint): GPT-2 XL's
// attention and MLP output projections (4096 x 1600 outputs, K = 1600 and
// 6400).  There 128 x 64 tiles make 800 workgroups for 1024 resident slots,
// so a quarter of the CUs hold a fourth tile while the rest hold three;
// 64 x 64 tiles make 1600, six or seven per CU (9.48 against 10.44 and
// 36.52 against 40.00 ms per step).  And its MLP input projection (4096 x
// 6400 outputs), where 128 x 64 tiles beat the model's 64 x 64 (32.9
// against 34.2 ms); for the QKV projection the model's 128 x 64 stayed
// faster than 64 x 64 (25.3 against 26.2 ms), and at 124M B = 4 the
// model's 128 x 128 for the MLP input projection than 64 x 64 (1.85
// against 2.15 ms).
int forward_tile(int N, int OC, int K) {
    struct Hint {
        int N, OC, K, tile;
    };
    static const Hint kHints[] = {{4096, 1600, 1600, 3}, {4096, 1600, 6400, 3}, {4096, 6400, 1600, 2}};
    for (const Hint &h : kHints)
        if (h.N == N && h.OC == OC && h.K == K) return h.tile;
    return plan_gemm(N, OC, K, 1, false).tile;
}

// out[N][OC] = inp[N][K] W^T (+ bias) with an epilogue.
hipError_t linear_fwd(float *out, const float *inp, const float *W, const float *bias, int N, int K, int OC,
                      int epi, const float *aux, float *out2, hipStream_t s) {
    GemmDesc d;
    d.a_kcontig = true; d.b_kcontig = true;
    d.M = N; d.N = OC; d.K = K;
    d.A = inp; d.lda = K; d.B = W; d.ldb = K; d.C = out; d.ldc = OC;
    d.epi = epi; d.bias = bias; d.aux = aux; d.ldaux = OC; d.C2 = out2;
    d.tile = forward_tile(N, OC, K);
    d.prec = g_prec;
    return gemm_run(d, s);
}

// Flops and compulsory bytes of one (unbatched, non-causal) product.
void gemm_cost(const GemmDesc &d, double &flops, double &bytes) {
    flops = 2.0 * d.M * d.N * d.K;
    double out = (double)d.M * d.N * (d.ksplit > 1 ? d.ksplit : 1);
    if (d.epi == EPI_ACCUM || d.epi == EPI_RESID || d.epi == EPI_GELU || d.epi == EPI_GELU_BWD) out *= 2;
    bytes = 4.0 * ((double)d.M * d.K + (double)d.K * d.N + out);
}

// Descriptors of the two products of a linear layer's backward.
// dinp[N][K] = dout[N][OC] W[OC][K] with epilogue epi (split-K partials to splitk if ks > 1)
GemmDesc dinp_desc(float *dinp, const float *dout, const float *W, int N, int K, int OC, int epi, const float *aux,
                   Plan p, float *splitk) {
    GemmDesc d;
    d.a_kcontig = true; d.b_kcontig = false;
    d.M = N; d.N = K; d.K = OC;
    d.A = dout; d.lda = OC; d.B = W; d.ldb = K; d.C = dinp; d.ldc = K;
    d.epi = epi; d.aux = aux; d.ldaux = K;
    d.tile = p.tile;
    d.prec = g_prec;
    if (p.ksplit > 1) { d.C = splitk; d.ksplit = p.ksplit; d.sCs = (long long)N * K; }
    return d;
}
// dW[OC][K] += dout^T inp, dbias += column sums of dout (partials to splitk / dbias_ws if ks > 1)
GemmDesc dw_desc(float *dW, float *dbias, const float *dout, const float *inp, int N, int K, int OC, Plan p,
                 float *splitk, float *dbias_ws) {
    GemmDesc d;
    d.a_kcontig = false; d.b_kcontig = false;
    d.M = OC; d.N = K; d.K = N;
    d.A = dout; d.lda = OC; d.B = inp; d.ldb = K; d.C = dW; d.ldc = K;
    d.tile = p.tile;
    d.prec = g_prec;
    if (p.ksplit > 1) {
        d.epi = EPI_STORE; d.C = splitk; d.ksplit = p.ksplit; d.sCs = (long long)OC * K;
        d.colsum = dbias ? dbias_ws : nullptr;
    } else {
        d.epi = EPI_ACCUM;
        d.colsum = dbias;
    }
    return d;
}

hipError_t dinp_finish(float *dinp, const float *splitk, int N, int K, int ks, hipStream_t s) {
    if (ks <= 1) return hipSuccess;
    return timed("sum_partials_kernel", 0, 4.0 * (ks + 1) * N * K,
                 [&]() { return k_sum_partials(dinp, splitk, ks, (size_t)N * K, false, s); });
}
hipError_t dw_finish(float *dW, float *dbias, const float *splitk, const float *dbias_ws, int K, int OC, int ks,
                     hipStream_t s) {
    if (ks <= 1) return hipSuccess;
    if (!dbias)
        return timed("sum_partials_kernel", 0, 4.0 * (ks + 2) * OC * K,
                     [&]() { return k_sum_partials(dW, splitk, ks, (size_t)OC * K, true, s); });
    return timed("sum_partials2_kernel", 0, 4.0 * (ks + 2) * ((double)OC * K + OC), [&]() {
        return k_sum_partials2(dW, splitk, (size_t)OC * K, dbias, dbias_ws, (size_t)OC, ks, true, s);
    });
}

// dinp[N][K] = dout[N][OC] W[OC][K] with an epilogue (the input gradient of a
// linear layer).  Split-K only for EPI_STORE and when splitk is given.
hipError_t linear_bwd_dinp(float *dinp, const float *dout, const float *W, int N, int K, int OC, int epi,
                           const float *aux, float *splitk, hipStream_t s) {
    const Plan p = plan_gemm(N, K, OC, 1, epi == EPI_STORE && splitk != nullptr);
    hipError_t e = gemm_run(dinp_desc(dinp, dout, W, N, K, OC, epi, aux, p, splitk), s);
    return e != hipSuccess ? e : dinp_finish(dinp, splitk, N, K, p.ksplit, s);
}

// dW[OC][K] += dout[N][OC]^T inp[N][K]; dbias[OC] += column sums of dout
// (dbias may be null).  With split-K the partial products go to `splitk`
// and the partial bias sums to `dbias_ws` (16 * OC floats).
hipError_t linear_bwd_dw(float *dW, float *dbias, const float *dout, const float *inp, int N, int K, int OC,
                         float *splitk, float *dbias_ws, hipStream_t s, bool defer_sum = false) {
    const Plan p = plan_gemm(OC, K, N, 1, splitk != nullptr);
    hipError_t e = gemm_run(dw_desc(dW, dbias, dout, inp, N, K, OC, p, splitk, dbias_ws), s);
    return e != hipSuccess || defer_sum ? e : dw_finish(dW, dbias, splitk, dbias_ws, K, OC, p.ksplit, s);
}

// Both gradients of a linear layer out = inp W^T + b given dout: the weight
// and bias gradients (accumulated) and the input gradient (with epilogue
// epi; dinp may be null to skip it).  When the planner predicts a gain the
// two products run as one grid, so that each fills the other's idle CUs.
// splitk_dinp (may be null: no split of the input gradient) and splitk_dw /
// dbias_ws are separate regions, both in use at once.
hipError_t linear_bwd(float *dinp, int epi, const float *aux, float *dW, float *dbias, const float *dout,
                      const float *inp, const float *W, int N, int K, int OC, float *splitk_dinp, float *splitk_dw,
                      float *dbias_ws, hipStream_t s, bool defer_dw_sum = false) {
    const bool split_dinp = epi == EPI_STORE && splitk_dinp != nullptr;
    const PairPlan pp = dinp ? plan_pair(N, K, OC, split_dinp) : PairPlan{false, 0, 1, 1};
    if (!pp.pair) {
        hipError_t e = dinp ? linear_bwd_dinp(dinp, dout, W, N, K, OC, epi, aux, splitk_dinp, s) : hipSuccess;
        return e != hipSuccess ? e
                               : linear_bwd_dw(dW, dbias, dout, inp, N, K, OC, splitk_dw, dbias_ws, s, defer_dw_sum);
    }
    const GemmDesc dd = dw_desc(dW, dbias, dout, inp, N, K, OC, Plan{pp.tile, pp.ks_dw}, splitk_dw, dbias_ws);
    const GemmDesc di = dinp_desc(dinp, dout, W, N, K, OC, epi, aux, Plan{pp.tile, pp.ks_dinp}, splitk_dinp);
    double f1, b1, f2, b2;
    gemm_cost(dd, f1, b1);
    gemm_cost(di, f2, b2);
    hipError_t e = timed(gemm_pair_kernel_name(pp.tile, gemm_pair_full(dd, di, pp.tile), dd.prec), f1 + f2, b1 + b2,
                         [&]() { return gemm_launch_pair(dd, di, s); });
    if (e == hipSuccess && !defer_dw_sum) e = dw_finish(dW, dbias, splitk_dw, dbias_ws, K, OC, pp.ks_dw, s);
    if (e == hipSuccess) e = dinp_finish(dinp, splitk_dinp, N, K, pp.ks_dinp, s);
    return e;
}

// Attention forward over qkv [B][T][3C]: att = softmax(scale Q K^T) (causal), atty = att V.
hipError_t attention_fwd(float *atty, float *att, const float *qkv, int B, int T, int C, int NH, hipStream_t s) {
    const int hd = C / NH;
    const long long C3 = 3LL * C, TT = (long long)T * T;
    GemmDesc d;
    d.a_kcontig = true; d.b_kcontig = true;
    d.M = T; d.N = T; d.K = hd;
    d.A = qkv; d.lda = C3; d.B = qkv + C; d.ldb = C3; d.C = att; d.ldc = T;
    d.alpha = 1.0f / sqrtf((float)hd);
    d.causal = CAUSAL_SKIP_UPPER;
    d.nbo = B; d.nbi = NH;
    d.sAo = T * C3; d.sAi = hd; d.sBo = T * C3; d.sBi = hd; d.sCo = NH * TT; d.sCi = TT;
    d.tile = plan_gemm(T, T, hd, (long long)B * NH, false).tile;
    hipError_t e = gemm_run(d, s, "attn_qk");
    if (e != hipSuccess) return e;
    const double tri = 0.5 * T * (T + 1.0) * B * NH;
    e = timed("attn_softmax_forward_kernel", 0, 8.0 * tri,
              [&]() { return k_attn_softmax_forward(att, (long long)B * NH * T, T, s); });
    if (e != hipSuccess) return e;
    GemmDesc y;
    y.a_kcontig = true; y.b_kcontig = false;
    y.M = T; y.N = hd; y.K = T;
    y.A = att; y.lda = T; y.B = qkv + 2 * C; y.ldb = C3; y.C = atty; y.ldc = C;
    y.causal = CAUSAL_KEND;
    y.nbo = B; y.nbi = NH;
    y.sAo = NH * TT; y.sAi = TT; y.sBo = T * C3; y.sBi = hd; y.sCo = (long long)T * C; y.sCi = hd;
    y.tile = plan_gemm(T, hd, T, (long long)B * NH, false).tile;
    return gemm_run(y, s, "attn_pv");
}

// Attention backward: dqkv (overwritten) from datty; dscore is B*NH*T*T scratch.
hipError_t attention_bwd(float *dqkv, float *dscore, const float *datty, const float *qkv, const float *att, int B,
                         int T, int C, int NH, hipStream_t s) {
    const int hd = C / NH;
    const long long C3 = 3LL * C, TT = (long long)T * T;
    const float scale = 1.0f / sqrtf((float)hd);
    const long long nb = (long long)B * NH;
    // dP = dY V^T on the causal tiles
    GemmDesc d;
    d.a_kcontig = true; d.b_kcontig = true;
    d.M = T; d.N = T; d.K = hd;
    d.A = datty; d.lda = C; d.B = qkv + 2 * C; d.ldb = C3; d.C = dscore; d.ldc = T;
    d.causal = CAUSAL_SKIP_UPPER;
    d.nbo = B; d.nbi = NH;
    d.sAo = (long long)T * C; d.sAi = hd; d.sBo = T * C3; d.sBi = hd; d.sCo = NH * TT; d.sCi = TT;
    d.tile = plan_gemm(T, T, hd, nb, false).tile;
    hipError_t e = gemm_run(d, s, "attn_dp");
    if (e != hipSuccess) return e;
    // dS = P (dP - rowsum(P dP)), in place
    const double tri = 0.5 * T * (T + 1.0) * nb;
    e = timed("attn_softmax_backward_kernel", 0, 12.0 * tri,
              [&]() { return k_attn_softmax_backward(dscore, att, nb * T, T, s); });
    if (e != hipSuccess) return e;
    // dQ = scale dS K
    GemmDesc q;
    q.a_kcontig = true; q.b_kcontig = false;
    q.M = T; q.N = hd; q.K = T;
    q.A = dscore; q.lda = T; q.B = qkv + C; q.ldb = C3; q.C = dqkv; q.ldc = C3;
    q.alpha = scale; q.causal = CAUSAL_KEND;
    q.nbo = B; q.nbi = NH;
    q.sAo = NH * TT; q.sAi = TT; q.sBo = T * C3; q.sBi = hd; q.sCo = T * C3; q.sCi = hd;
    q.tile = plan_gemm(T, hd, T, nb, false).tile;
    e = gemm_run(q, s, "attn_dq");
    if (e != hipSuccess) return e;
    // dK = scale dS^T Q
    GemmDesc k = q;
    k.a_kcontig = false; k.b_kcontig = false;
    k.B = qkv; k.C = dqkv + C; k.causal = CAUSAL_KSTART;
    e = gemm_run(k, s, "attn_dk");
    if (e != hipSuccess) return e;
    // dV = P^T dY
    GemmDesc v = k;
    v.A = att; v.alpha = 1.0f;
    v.B = datty; v.ldb = C; v.sBo = (long long)T * C; v.sBi = hd;
    v.C = dqkv + 2 * C;
    return gemm_run(v, s, "attn_dv");
}

// Fused attention backward: D, dk, dv and ds in the attention kernels, then
// dq = scale ds K as a causal GEMM over the ds matrices.
hipError_t flash_backward(float *dqkv, float *Dbuf, float *ws, const float *datty, const float *qkv,
                          const float *atty, const float *lse, int B, int T, int C, int NH, hipStream_t s) {
    const int hd = C / NH;
    const double tri = 0.5 * T * (T + 1.0) * B * NH;
    const size_t BTC = (size_t)B * T * C;
    // counted: dp, dv, dk (the recomputed s is not)
    hipError_t e = timed(flash_name(FL_DKDV, hd), 6.0 * tri * hd, 24.0 * BTC + 4.0 * tri, [&]() {
        return flash_attention_backward_dkdv(dqkv, ws, Dbuf, datty, qkv, atty, lse, B, T, C, NH, s);
    });
    if (e != hipSuccess) return e;
    // ds rows are Tp floats apart, zero past T
    const long long C3 = 3LL * C, Tp = (T + 3) / 4 * 4, TT = (long long)T * Tp;
    GemmDesc q;
    q.a_kcontig = true; q.b_kcontig = false; q.a_kpad = true;
    q.M = T; q.N = hd; q.K = T;
    q.A = flash_attention_ds(ws); q.lda = Tp; q.B = qkv + C; q.ldb = C3; q.C = dqkv; q.ldc = C3;
    q.alpha = 1.0f / sqrtf((float)hd); q.causal = CAUSAL_KEND;
    q.nbo = B; q.nbi = NH;
    q.sAo = NH * TT; q.sAi = TT; q.sBo = T * C3; q.sBi = hd; q.sCo = T * C3; q.sCi = hd;
    q.tile = plan_gemm(T, hd, T, (long long)B * NH, false).tile;
    // each folded pair of row tiles as two workgroups: few row tiles per head
    q.part = flash_attention_dq_partial(ws, B, T, NH);
    return gemm_run(q, s, "attn_dq");
}

}  // namespace

// ====================================================================== C ABI

extern "C" {

gpt2_status gpt2_query_sizes(const gpt2_config *cfg, int B, int T, gpt2_sizes *out) {
    std::string why;
    if (!config_ok(cfg, B, T, &why)) return fail(nullptr, GPT2_EINVAL, why);
    if (!out) return fail(nullptr, GPT2_EINVAL, "out is NULL");
    Layout l;
    make_layout(cfg, B, T, &l);
    out->params = l.nparams;
    out->acts = l.nacts;
    out->work = l.nwork;
    out->iwork = l.niwork;
    return GPT2_OK;
}

gpt2_status gpt2_layout(const gpt2_config *cfg, int B, int T, int which, int idx, const char **name,
                        size_t *offset, size_t *count) {
    std::string why;
    if (!config_ok(cfg, B, T, &why)) return fail(nullptr, GPT2_EINVAL, why);
    Layout l;
    make_layout(cfg, B, T, &l);
    if (which == GPT2_PARAMS && idx >= 0 && idx < 16) {
        if (name) *name = kParamNames[idx];
        if (offset) *offset = l.poff[idx];
        if (count) *count = l.pcnt[idx];
        return GPT2_OK;
    }
    if (which == GPT2_ACTS && idx >= 0 && idx < NUM_ACTS) {
        if (name) *name = kActNames[idx];
        if (offset) *offset = l.aoff[idx];
        if (count) *count = l.acnt[idx];
        return GPT2_OK;
    }
    return fail(nullptr, GPT2_EINVAL, "layout index out of range");
}

gpt2_status gpt2_build(const gpt2_config *cfg, int B, int T, const gpt2_buffers *dev,
                       const float *init_params_host, void *hip_stream, gpt2_model **out) {
    std::string why;
    if (!out) return fail(nullptr, GPT2_EINVAL, "out is NULL");
    *out = nullptr;
    if (!config_ok(cfg, B, T, &why)) return fail(nullptr, GPT2_EINVAL, why);
    if (!dev || !dev->params || !dev->grads || !dev->adam_m || !dev->adam_v || !dev->acts || !dev->work ||
        !dev->iwork)
        return fail(nullptr, GPT2_EINVAL, "a device buffer is NULL");
    const void *ptrs[7] = {dev->params, dev->grads, dev->adam_m, dev->adam_v, dev->acts, dev->work, dev->iwork};
    for (const void *p : ptrs)
        if ((uintptr_t)p & 255) return fail(nullptr, GPT2_EINVAL, "device buffers must be 256-byte aligned");
    gpt2_model *m = new gpt2_model();
    make_layout(cfg, B, T, &m->lo);
    m->buf = *dev;
    m->stream = (hipStream_t)hip_stream;
    const size_t np = m->lo.nparams;
    hipError_t e = hipSuccess;
    if (init_params_host) {
        e = hipMemcpyAsync(dev->params, init_params_host, np * sizeof(float), hipMemcpyHostToDevice, m->stream);
        if (e == hipSuccess) e = hipStreamSynchronize(m->stream);
    }
    if (e == hipSuccess) e = k_fill(dev->grads, np, 0.0f, m->stream);
    if (e == hipSuccess) e = k_fill(dev->adam_m, np, 0.0f, m->stream);
    if (e == hipSuccess) e = k_fill(dev->adam_v, np, 0.0f, m->stream);
    if (e == hipSuccess) e = k_fill_i32(dev->iwork, m->lo.niwork, 0, m->stream);
    if (e != hipSuccess) {
        std::string msg = std::string("gpt2_build: ") + hipGetErrorString(e);
        gpt2_free(m);
        return fail(nullptr, GPT2_EDEVICE, msg);
    }
    *out = m;
    return GPT2_OK;
}

gpt2_status gpt2_forward(gpt2_model *m, const int32_t *inputs, const int32_t *targets, float *mean_loss) {
    if (!m) return fail(nullptr, GPT2_EINVAL, "model is NULL");
    ProfScope prof_scope(m);
    PrecScope prec_scope(m->mm_prec);
    if (!inputs) return fail(m, GPT2_EINVAL, "inputs is NULL");
    if (mean_loss && !targets) return fail(m, GPT2_EINVAL, "mean_loss needs targets");
    const Layout &l = m->lo;
    const int B = l.B, T = l.T, C = l.C, NH = l.NH, BT = (int)l.BT;
    const size_t BTC = (size_t)BT * C;
    hipStream_t s = m->stream;
    float *P = m->buf.params, *A = m->buf.acts;
    int32_t *order = m->buf.iwork + l.i_order, *err = m->buf.iwork + l.i_err;
    int32_t *tok = m->buf.iwork + l.i_tok;
    m->have_targets = false;

    // keep this batch's ids for the embedding backward
    HIPCK(m, copy_ids(tok, inputs, BT, s));
    inputs = tok;
    KRUN(m, k_token_prep_name(BT), 12.0 * BT, k_token_prep(inputs, targets, order, err, m->buf.iwork + l.i_sort, BT, l.V, s));
    KRUN(m, "encoder_forward_kernel", 12.0 * BTC, k_encoder_forward(A + l.aoff[A_ENCODED], inputs, P + l.poff[0], P + l.poff[1], B, T, C, l.V, s));
    for (int li = 0; li < l.L; li++) {
        const float *res = li == 0 ? A + l.aoff[A_ENCODED] : A + l.aoff[A_RES3] + (li - 1) * BTC;
        float *ln1 = A + l.aoff[A_LN1] + li * BTC;
        float *ln1m = A + l.aoff[A_LN1_MEAN] + (size_t)li * BT, *ln1r = A + l.aoff[A_LN1_RSTD] + (size_t)li * BT;
        float *qkv = A + l.aoff[A_QKV] + li * 3 * BTC;
        float *att = A + l.aoff[A_ATT] + (size_t)li * B * NH * T * T;
        float *atty = A + l.aoff[A_ATTY] + li * BTC;
        float *res2 = A + l.aoff[A_RES2] + li * BTC;
        float *ln2 = A + l.aoff[A_LN2] + li * BTC;
        float *ln2m = A + l.aoff[A_LN2_MEAN] + (size_t)li * BT, *ln2r = A + l.aoff[A_LN2_RSTD] + (size_t)li * BT;
        float *fch = A + l.aoff[A_FCH] + li * 4 * BTC, *fchg = A + l.aoff[A_FCH_GELU] + li * 4 * BTC;
        float *res3 = A + l.aoff[A_RES3] + li * BTC;
        const size_t c = C;
        KRUN(m, "layernorm_forward_kernel", 8.0 * (BTC + BT), k_layernorm_forward(ln1, ln1m, ln1r, res, P + l.poff[2] + li * c, P + l.poff[3] + li * c, BT, C, s));
        {
            Site site_("qkv");
            HIPCK(m, linear_fwd(qkv, ln1, P + l.poff[4] + li * 3 * c * c, P + l.poff[5] + li * 3 * c, BT, C, 3 * C,
                            EPI_STORE, nullptr, nullptr, s));
        }
        if (l.flash) {
            float *lse = A + l.aoff[A_LSE] + (size_t)li * B * NH * T;
            const double tri = 0.5 * T * (T + 1.0) * B * NH;
            KRUNF(m, flash_name(FL_FWD, l.hd), 4.0 * tri * l.hd, 16.0 * BTC,
                 flash_attention_forward(atty, lse, m->buf.work + l.w_flash, qkv, B, T, C, NH, s));
        } else {
            Site site_("attn_fwd");
            HIPCK(m, attention_fwd(atty, att, qkv, B, T, C, NH, s));
        }
        {
            Site site_("attproj");
            HIPCK(m, linear_fwd(res2, atty, P + l.poff[6] + li * c * c, P + l.poff[7] + li * c, BT, C, C, EPI_RESID,
                            res, nullptr, s));
        }
        KRUN(m, "layernorm_forward_kernel", 8.0 * (BTC + BT), k_layernorm_forward(ln2, ln2m, ln2r, res2, P + l.poff[8] + li * c, P + l.poff[9] + li * c, BT, C, s));
        {
            Site site_("fc");
            HIPCK(m, linear_fwd(fch, ln2, P + l.poff[10] + li * 4 * c * c, P + l.poff[11] + li * 4 * c, BT, C, 4 * C,
                            EPI_GELU, nullptr, fchg, s));
        }
        {
            Site site_("fcproj");
            HIPCK(m, linear_fwd(res3, fchg, P + l.poff[12] + li * 4 * c * c, P + l.poff[13] + li * c, BT, 4 * C, C,
                            EPI_RESID, res2, nullptr, s));
        }
    }
    const float *last = A + l.aoff[A_RES3] + (size_t)(l.L - 1) * BTC;
    float *lnf = A + l.aoff[A_LNF], *logits = A + l.aoff[A_LOGITS];
    KRUN(m, "layernorm_forward_kernel", 8.0 * (BTC + BT), k_layernorm_forward(lnf, A + l.aoff[A_LNF_MEAN], A + l.aoff[A_LNF_RSTD], last, P + l.poff[14],
                                 P + l.poff[15], BT, C, s));
    {
        Site site_("head");
        HIPCK(m, linear_fwd(logits, lnf, P + l.poff[0], nullptr, BT, C, l.Vp, EPI_STORE, nullptr, nullptr, s));
    }
    if (targets) {
        KRUN(m, k_crossentropy_name(l.Vp), 8.0 * BT * l.Vp, k_crossentropy(logits, A + l.aoff[A_LOSSES], targets, BT, l.V, l.Vp, 1.0f / BT, err, s));
        KRUN(m, "mean_kernel", 4.0 * BT, k_mean(A + l.aoff[A_LOSS], A + l.aoff[A_LOSSES], BT, s));
        m->have_targets = true;
    }
    if (mean_loss) {
        float h_loss = 0.f;
        int32_t h_err = 0;
        HIPCK(m, hipMemcpyAsync(&h_loss, A + l.aoff[A_LOSS], sizeof(float), hipMemcpyDeviceToHost, s));
        HIPCK(m, hipMemcpyAsync(&h_err, err, sizeof(int32_t), hipMemcpyDeviceToHost, s));
        HIPCK(m, hipStreamSynchronize(s));
        *mean_loss = h_loss;
        if (h_err) {
            HIPCK(m, k_fill_i32(err, 1, 0, s));
            m->have_targets = false;  // this batch's loss gradient is zero and may not be used
            return fail(m, GPT2_ERANGE, h_err & 1 ? "an input id is outside [0, vocab_size)"
                                                  : "a target id is outside [0, vocab_size)");
        }
    }
    return GPT2_OK;
}

gpt2_status gpt2_zero_grad(gpt2_model *m) {
    if (!m) return fail(nullptr, GPT2_EINVAL, "model is NULL");
    ProfScope prof_scope(m);
    KRUN(m, "fill4_kernel", 4.0 * m->lo.nparams, k_fill(m->buf.grads, m->lo.nparams, 0.0f, m->stream));
    return GPT2_OK;
}

gpt2_status gpt2_backward(gpt2_model *m) {
    if (!m) return fail(nullptr, GPT2_EINVAL, "model is NULL");
    ProfScope prof_scope(m);
    PrecScope prec_scope(m->mm_prec);
    if (!m->have_targets) return fail(m, GPT2_ESTATE, "gpt2_backward needs a preceding gpt2_forward with targets");
    const Layout &l = m->lo;
    const int B = l.B, T = l.T, C = l.C, NH = l.NH, BT = (int)l.BT;
    const size_t BTC = (size_t)BT * C, c = C;
    hipStream_t s = m->stream;
    float *P = m->buf.params, *G = m->buf.grads, *A = m->buf.acts, *W = m->buf.work;
    float *dres = W + l.w_dres, *dln = W + l.w_dln, *datty = W + l.w_datty, *dqkv = W + l.w_dqkv;
    float *dfch = W + l.w_dfch, *dscore = W + l.w_datt, *part = W + l.w_part, *splitk = W + l.w_splitk;
    float *splitk_dw = W + l.w_splitk_dw, *dbias_ws = W + l.w_dbias;
    const float *dlogits = A + l.aoff[A_LOGITS], *lnf = A + l.aoff[A_LNF];
    // per-site split-K partials of layer li (their sums for all layers come at the end)
    const int s_in[NSITES] = {C, C, C, 4 * C}, s_out[NSITES] = {3 * C, C, 4 * C, C};
    auto site_dw = [&](int j, int li) {
        return l.site_ks[j] > 1 ? W + l.w_site_dw[j] + (size_t)li * l.site_ks[j] * s_out[j] * s_in[j] : splitk_dw;
    };
    auto site_db = [&](int j, int li) {
        return l.site_ks[j] > 1 ? W + l.w_site_db[j] + (size_t)li * l.site_ks[j] * s_out[j] : dbias_ws;
    };

    // head: dlnf = dlogits wte, dwte += dlogits^T lnf
    {
        Site site_("head_bwd");
        HIPCK(m, linear_bwd(dln, EPI_STORE, nullptr, G + l.poff[0], nullptr, dlogits, lnf, P + l.poff[0], BT, C, l.Vp,
                            splitk, splitk_dw, dbias_ws, s));
    }
    const float *last = A + l.aoff[A_RES3] + (size_t)(l.L - 1) * BTC;
    const size_t pslot = (size_t)ln_partials(BT) * 2 * C;  // floats of one LayerNorm's partials
    KRUN(m, "layernorm_backward_kernel", 12.0 * BTC, k_layernorm_backward(dres, nullptr, nullptr, part + 2 * l.L * pslot, dln, last, P + l.poff[14],
                                  A + l.aoff[A_LNF_MEAN], A + l.aoff[A_LNF_RSTD], BT, C, false, s));
    for (int li = l.L - 1; li >= 0; li--) {
        const float *res = li == 0 ? A + l.aoff[A_ENCODED] : A + l.aoff[A_RES3] + (li - 1) * BTC;
        const float *ln1 = A + l.aoff[A_LN1] + li * BTC;
        const float *ln1m = A + l.aoff[A_LN1_MEAN] + (size_t)li * BT, *ln1r = A + l.aoff[A_LN1_RSTD] + (size_t)li * BT;
        const float *qkv = A + l.aoff[A_QKV] + li * 3 * BTC;
        const float *att = A + l.aoff[A_ATT] + (size_t)li * B * NH * T * T;
        const float *atty = A + l.aoff[A_ATTY] + li * BTC;
        const float *res2 = A + l.aoff[A_RES2] + li * BTC;
        const float *ln2 = A + l.aoff[A_LN2] + li * BTC;
        const float *ln2m = A + l.aoff[A_LN2_MEAN] + (size_t)li * BT, *ln2r = A + l.aoff[A_LN2_RSTD] + (size_t)li * BT;
        const float *fch = A + l.aoff[A_FCH] + li * 4 * BTC, *fchg = A + l.aoff[A_FCH_GELU] + li * 4 * BTC;
        const float *qkvw = P + l.poff[4] + li * 3 * c * c, *aw = P + l.poff[6] + li * c * c;
        const float *fw = P + l.poff[10] + li * 4 * c * c, *pw = P + l.poff[12] + li * 4 * c * c;

        // fcproj: dout = dres (gradient of residual3); dfch through GELU'
        {
            Site site_("fcproj_bwd");
            HIPCK(m, linear_bwd(dfch, EPI_GELU_BWD, fch, G + l.poff[12] + li * 4 * c * c, G + l.poff[13] + li * c, dres,
                                fchg, pw, BT, 4 * C, C, nullptr, site_dw(SITE_FCPROJ, li), site_db(SITE_FCPROJ, li), s,
                                true));
        }
        // fc
        {
            Site site_("fc_bwd");
            HIPCK(m, linear_bwd(dln, EPI_STORE, nullptr, G + l.poff[10] + li * 4 * c * c, G + l.poff[11] + li * 4 * c,
                                dfch, ln2, fw, BT, C, 4 * C, nullptr, site_dw(SITE_FC, li), site_db(SITE_FC, li), s, true));
        }
        // ln2: dres becomes the gradient of residual2
        KRUN(m, "layernorm_backward_kernel", 16.0 * BTC, k_layernorm_backward(dres, nullptr, nullptr, part + (l.L + li) * pslot, dln, res2,
                                      P + l.poff[8] + li * c, ln2m, ln2r, BT, C, true, s));
        // attproj: dout = dres
        {
            Site site_("attproj_bwd");
            HIPCK(m, linear_bwd(datty, EPI_STORE, nullptr, G + l.poff[6] + li * c * c, G + l.poff[7] + li * c, dres,
                                atty, aw, BT, C, C, nullptr, site_dw(SITE_ATTPROJ, li), site_db(SITE_ATTPROJ, li), s,
                                true));
        }
        // attention
        if (l.flash) {
            const float *lse = A + l.aoff[A_LSE] + (size_t)li * B * NH * T;
            HIPCK(m, flash_backward(dqkv, dscore, W + l.w_flash, datty, qkv, atty, lse, B, T, C, NH, s));
        } else {
            Site site_("attn_bwd");
            HIPCK(m, attention_bwd(dqkv, dscore, datty, qkv, att, B, T, C, NH, s));
        }
        // qkv
        {
            Site site_("qkv_bwd");
            HIPCK(m, linear_bwd(dln, EPI_STORE, nullptr, G + l.poff[4] + li * 3 * c * c, G + l.poff[5] + li * 3 * c, dqkv,
                                ln1, qkvw, BT, C, 3 * C, nullptr, site_dw(SITE_QKV, li), site_db(SITE_QKV, li), s, true));
        }
        // ln1: dres becomes the gradient of this layer's input
        KRUN(m, "layernorm_backward_kernel", 16.0 * BTC, k_layernorm_backward(dres, nullptr, nullptr, part + li * pslot, dln, res,
                                      P + l.poff[2] + li * c, ln1m, ln1r, BT, C, true, s));
    }
    // weight and bias gradients of the split sites, all layers of a site in one launch
    {
        const int pw_[NSITES] = {4, 6, 10, 12};
        for (int j = 0; j < NSITES; j++) {
            const int ks = l.site_ks[j];
            if (ks <= 1) continue;
            const size_t n1 = (size_t)s_out[j] * s_in[j], n2 = (size_t)s_out[j];
            KRUN(m, "sum_layers_kernel", 4.0 * (ks + 2) * (double)l.L * (n1 + n2),
                 k_sum_layers(G + l.poff[pw_[j]], W + l.w_site_dw[j], n1, G + l.poff[pw_[j] + 1], W + l.w_site_db[j], n2,
                              ks, l.L, s));
        }
    }
    // gamma / beta gradients of every LayerNorm from their partials, one launch
    KRUN(m, "ln_param_sums_kernel", 4.0 * (2 * l.L + 1) * (pslot + 4.0 * C),
         k_ln_param_sums(G + l.poff[2], G + l.poff[3], G + l.poff[8], G + l.poff[9], G + l.poff[14], G + l.poff[15], l.L,
                         part, BT, C, s));
    // (datty is free by now: it holds the segment sums of the embedding scatter-add)
    KRUN(m, "encoder_backward_kernel", 16.0 * BTC, k_encoder_backward(G + l.poff[0], G + l.poff[1], datty, dres, m->buf.iwork + l.i_tok, m->buf.iwork + l.i_order, B, T, C,
                                l.V, s));
    return GPT2_OK;
}

gpt2_status gpt2_update(gpt2_model *m, float lr, float beta1, float beta2, float eps, float weight_decay, int t) {
    if (!m) return fail(nullptr, GPT2_EINVAL, "model is NULL");
    ProfScope prof_scope(m);
    if (t < 1) return fail(m, GPT2_EINVAL, "t must be >= 1");
    double c1 = 1.0 - std::pow((double)beta1, t), c2 = 1.0 - std::pow((double)beta2, t);
    KRUN(m, "adamw_kernel", 28.0 * m->lo.nparams, k_adamw(m->buf.params, m->buf.grads, m->buf.adam_m, m->buf.adam_v, m->lo.nparams, lr, beta1, beta2,
                     eps, weight_decay, (float)c1, (float)c2, m->buf.iwork + m->lo.i_err, m->stream));
    return GPT2_OK;
}

namespace {

// The launches of one decoding step on stream s, for the position in the
// model's device int (set before, by gpt2_decode_step).
// pos: the position decoded, for the byte counts of per-launch profiling
// only (the kernels read it from the device, so that a captured step serves
// every position).
gpt2_status decode_launches(gpt2_model *m, hipStream_t s, const int32_t *tokens, const float *coins, int32_t *next,
                            int pos) {
    const Layout &l = m->lo;
    const int B = l.B, T = l.T, C = l.C, NH = l.NH;
    const size_t BTC = (size_t)l.BT * C, c = C;
    float *P = m->buf.params, *A = m->buf.acts;
    float *x = m->buf.work + l.w_dec, *att = x + (size_t)B * C, *h = att + (size_t)B * C;
    float *aws = h + (size_t)4 * B * C;
    int32_t *err = m->buf.iwork + l.i_err;
    const int *dpos = m->buf.iwork + l.i_dec;
    const double w = 4.0 * B;  // bytes per float of one row per sequence
    KRUN(m, "decode_embed_kernel", 3.0 * w * C, k_decode_embed(x, tokens, P + l.poff[0], P + l.poff[1], dpos, err, B, C, l.V, T, s));
    for (int li = 0; li < l.L; li++) {
        float *qkv = A + l.aoff[A_QKV] + li * 3 * BTC;  // this layer's cache: rows (b, u) of q | k | v
        // the new rows' q | k | v from LayerNorm(x) (computed inside), at row (b, pos)
        KRUNF(m, k_rows_linear_name(C), 2.0 * B * C * 3 * C, 4.0 * 3 * C * C + w * 4 * C,
              k_rows_linear(qkv, (long long)T * 3 * C, x, C, P + l.poff[4] + li * 3 * c * c, P + l.poff[5] + li * 3 * c,
                            nullptr, 0, P + l.poff[2] + li * c, P + l.poff[3] + li * c, B, C, 3 * C, 0, dpos, 3 * C,
                            T - 1, s));
        KRUN(m, "decode_attn_partial_kernel", w * C * 2.0 * (pos + 1),  // k and v rows u <= pos
             k_decode_attention(att, aws, qkv, dpos, B, T, C, NH, s));
        KRUNF(m, k_rows_linear_name(C), 2.0 * B * C * C, 4.0 * C * C + 3 * w * C,
              k_rows_linear(x, C, att, C, P + l.poff[6] + li * c * c, P + l.poff[7] + li * c, x, C, nullptr, nullptr, B,
                            C, C, 1, nullptr, 0, 0, s));
        KRUNF(m, k_rows_linear_name(C), 2.0 * B * C * 4 * C, 4.0 * 4 * C * C + w * 5 * C,
              k_rows_linear(h, 4 * C, x, C, P + l.poff[10] + li * 4 * c * c, P + l.poff[11] + li * 4 * c, nullptr, 0,
                            P + l.poff[8] + li * c, P + l.poff[9] + li * c, B, C, 4 * C, 2, nullptr, 0, 0, s));
        KRUNF(m, k_rows_linear_name(4 * C), 2.0 * B * 4 * C * C, 4.0 * 4 * C * C + w * 6 * C,
              k_rows_linear(x, C, h, 4 * C, P + l.poff[12] + li * 4 * c * c, P + l.poff[13] + li * c, x, C, nullptr,
                            nullptr, B, 4 * C, C, 1, nullptr, 0, 0, s));
    }
    float *logits = A + l.aoff[A_LOGITS];  // row (b, pos) at (b T + pos) Vp
    KRUNF(m, k_rows_linear_name(C), 2.0 * B * C * l.Vp, 4.0 * (double)l.Vp * C + w * (C + l.Vp),
          k_rows_linear(logits, (long long)T * l.Vp, x, C, P + l.poff[0], nullptr, nullptr, 0, P + l.poff[14],
                        P + l.poff[15], B, C, l.Vp, 0, dpos, l.Vp, T - 1, s));
    KRUN(m, "sample_kernel", w * l.V, k_sample(next, logits, (long long)T * l.Vp, B, l.V, coins, dpos, l.Vp, T - 1, s));
    return GPT2_OK;
}

// The decoding step for (tokens, coins, next) captured into a graph on a
// stream of the model's own (the launches only record device pointers, and
// the position is read from the device), or null if capture failed.
hipGraphExec_t decode_graph(gpt2_model *m, const int32_t *tokens, const float *coins, int32_t *next) {
    for (const auto &g : m->decode_graphs)
        if (g.tokens == tokens && g.coins == coins && g.next == next) return g.exec;
    if (!m->graphs_ok) return nullptr;
    if (m->decode_graphs.size() >= 8) {  // a few argument sets are in use at a time
        for (auto &g : m->decode_graphs) (void)hipGraphExecDestroy(g.exec);
        m->decode_graphs.clear();
    }
    if (!m->capture_stream && hipStreamCreateWithFlags(&m->capture_stream, hipStreamNonBlocking) != hipSuccess) {
        m->capture_stream = nullptr;
        m->graphs_ok = false;
        return nullptr;
    }
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    bool ok = hipStreamBeginCapture(m->capture_stream, hipStreamCaptureModeThreadLocal) == hipSuccess;
    if (ok) {
        const gpt2_status st = decode_launches(m, m->capture_stream, tokens, coins, next, m->lo.T - 1);
        ok = hipStreamEndCapture(m->capture_stream, &graph) == hipSuccess && st == GPT2_OK && graph;
    }
    if (ok) ok = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) == hipSuccess;
    if (graph) (void)hipGraphDestroy(graph);
    if (!ok) {
        (void)hipGetLastError();
        m->graphs_ok = false;  // direct launches from now on
        return nullptr;
    }
    m->decode_graphs.push_back({tokens, coins, next, exec});
    return exec;
}

}  // namespace

gpt2_status gpt2_decode_step(gpt2_model *m, const int32_t *tokens, int pos, const float *coins, int32_t *next) {
    if (!m) return fail(nullptr, GPT2_EINVAL, "model is NULL");
    ProfScope prof_scope(m);
    if (!tokens || !next) return fail(m, GPT2_EINVAL, "tokens and next are required");
    const Layout &l = m->lo;
    if (pos < 0 || pos >= l.T) return fail(m, GPT2_EINVAL, "pos must be in [0, T)");
    hipStream_t s = m->stream;
    m->have_targets = false;  // rows of the saved activations are overwritten
    // the position, for every kernel of the step (its own launch, so that a
    // captured step serves every position)
    KRUN(m, "set_int_kernel", 4.0, k_set_int(m->buf.iwork + l.i_dec, pos, s));
    if (!m->prof.on && !audit_sink()) {
        if (hipGraphExec_t exec = decode_graph(m, tokens, coins, next)) {
            HIPCK(m, hipGraphLaunch(exec, s));
            return GPT2_OK;
        }
    }
    return decode_launches(m, s, tokens, coins, next, pos);
}

gpt2_status gpt2_set_matmul_precision(gpt2_model *m, int precision) {
    if (!m) return fail(nullptr, GPT2_EINVAL, "model is NULL");
    if (precision != GPT2_FP32 && precision != GPT2_BF16) return fail(m, GPT2_EINVAL, "unknown precision");
    m->mm_prec = precision;
    return GPT2_OK;
}

gpt2_status gpt2_sync(gpt2_model *m) {
    if (!m) return fail(nullptr, GPT2_EINVAL, "model is NULL");
    int32_t h_err = 0;
    HIPCK(m, hipMemcpyAsync(&h_err, m->buf.iwork + m->lo.i_err, sizeof(int32_t), hipMemcpyDeviceToHost, m->stream));
    HIPCK(m, hipStreamSynchronize(m->stream));
    if (h_err) {
        HIPCK(m, k_fill_i32(m->buf.iwork + m->lo.i_err, 1, 0, m->stream));
        m->have_targets = false;
        return fail(m, GPT2_ERANGE, "an id was outside [0, vocab_size)");
    }
    return GPT2_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- checkpoints
// (file format in checkpoint.h; here the copies between the device and the
// host staging buffer)
namespace {

CkModel ck_model(const Layout &l) {
    CkModel c;
    const int32_t cfg[6] = {l.maxT, l.V, l.Vp, l.L, l.NH, l.C};
    memcpy(c.cfg, cfg, sizeof cfg);
    c.nparams = (int64_t)l.nparams;
    for (int i = 0; i < 16; i++) {
        c.names[i] = kParamNames[i];
        c.offset[i] = (int64_t)l.poff[i];
        c.count[i] = (int64_t)l.pcnt[i];
    }
    return c;
}

gpt2_status ck_status(gpt2_model *m, int code, const std::string &msg, hipError_t e) {
    if (code == CK_OK) return GPT2_OK;
    if (code == CK_ECOPY) return fail(m, GPT2_EDEVICE, msg + ": " + hipGetErrorString(e));
    return fail(m, code == CK_EINVAL ? GPT2_EINVAL : GPT2_EIO, msg);
}

}  // namespace

extern "C" {

gpt2_status gpt2_save_checkpoint(gpt2_model *m, const char *path, int t) {
    if (!m) return fail(nullptr, GPT2_EINVAL, "model is NULL");
    HIPCK(m, hipStreamSynchronize(m->stream));  // the state on the device is complete
    const float *src[3] = {m->buf.params, m->buf.adam_m, m->buf.adam_v};
    hipError_t e = hipSuccess;
    auto fetch = [&](int a, size_t first, size_t count, float *dst) {
        e = hipMemcpyAsync(dst, src[a] + first, count * sizeof(float), hipMemcpyDeviceToHost, m->stream);
        if (e == hipSuccess) e = hipStreamSynchronize(m->stream);
        return e == hipSuccess ? 0 : 1;
    };
    std::string msg;
    const int code = ck_save(path, ck_model(m->lo), t, fetch, &msg);
    return ck_status(m, code, msg, e);
}

gpt2_status gpt2_load_checkpoint(gpt2_model *m, const char *path, int *t) {
    if (!m) return fail(nullptr, GPT2_EINVAL, "model is NULL");
    HIPCK(m, hipStreamSynchronize(m->stream));
    float *dst[3] = {m->buf.params, m->buf.adam_m, m->buf.adam_v};
    hipError_t e = hipSuccess;
    auto store = [&](int a, size_t first, size_t count, const float *src) {
        e = hipMemcpyAsync(dst[a] + first, src, count * sizeof(float), hipMemcpyHostToDevice, m->stream);
        if (e == hipSuccess) e = hipStreamSynchronize(m->stream);
        return e == hipSuccess ? 0 : 1;
    };
    std::string msg;
    const int code = ck_load(path, ck_model(m->lo), t, store, &msg);
    if (code == CK_OK || code == CK_ECOPY) m->have_targets = false;  // activations belong to the old parameters
    return ck_status(m, code, msg, e);
}

gpt2_status gpt2_profile_enable(gpt2_model *m, int enable) {
    if (!m) return fail(nullptr, GPT2_EINVAL, "model is NULL");
    m->prof.on = enable != 0;
    m->prof.stream = m->stream;
    // create events up front so that none is created inside a timed region
    while (m->prof.on && m->prof.pool.size() < 4096) {
        hipEvent_t e;
        HIPCK(m, hipEventCreate(&e));
        m->prof.pool.push_back(e);
    }
    return GPT2_OK;
}

gpt2_status gpt2_profile_read(gpt2_model *m, gpt2_profile_entry *out, int max_entries, int *n_entries) {
    if (!m) return fail(nullptr, GPT2_EINVAL, "model is NULL");
    HIPCK(m, hipStreamSynchronize(m->stream));
    std::vector<gpt2_profile_entry> agg;
    for (const ProfRec &r : m->prof.recs) {
        float ms = 0.f;
        HIPCK(m, hipEventElapsedTime(&ms, r.a, r.b));
        char key[sizeof(gpt2_profile_entry::name)];
        snprintf(key, sizeof key, "%s|%s", r.name, r.site);
        gpt2_profile_entry *e = nullptr;
        for (auto &x : agg)
            if (strncmp(x.name, key, sizeof x.name) == 0) e = &x;
        if (!e) {
            agg.push_back(gpt2_profile_entry{});
            e = &agg.back();
            strncpy(e->name, key, sizeof e->name - 1);
        }
        e->launches += 1;
        e->ms += ms;
        e->flops += r.flops;
        e->bytes += r.bytes;
    }
    m->prof.recs.clear();
    m->prof.used = 0;
    int n = (int)agg.size();
    if (n_entries) *n_entries = n;
    for (int i = 0; i < n && i < max_entries && out; i++) out[i] = agg[i];
    return GPT2_OK;
}

void gpt2_free(gpt2_model *m) {
    if (!m) return;
    for (auto &g : m->decode_graphs) (void)hipGraphExecDestroy(g.exec);
    if (m->capture_stream) (void)hipStreamDestroy(m->capture_stream);
    for (hipEvent_t e : m->prof.pool) (void)hipEventDestroy(e);
    delete m;
}

const char *gpt2_last_error(const gpt2_model *m) { return m ? m->err.c_str() : g_last_error.c_str(); }

// ====================================================================== kernel-level entry points

#define KCK(expr)                                                                                      \
    do {                                                                                               \
        hipError_t e_ = (expr);                                                                        \
        if (e_ == hipErrorInvalidValue) return fail(nullptr, GPT2_EINVAL, std::string(#expr) + ": invalid shape or alignment"); \
        if (e_ != hipSuccess) return fail(nullptr, GPT2_EDEVICE, std::string(#expr) + ": " + hipGetErrorString(e_)); \
    } while (0)

gpt2_status gpt2k_linear_forward(float *out, const float *inp, const float *W, const float *bias, int N, int K,
                                 int OC, void *stream) {
    return gpt2k_linear_forward_prec(out, inp, W, bias, N, K, OC, GPT2_FP32, stream);
}

gpt2_status gpt2k_linear_forward_prec(float *out, const float *inp, const float *W, const float *bias, int N, int K,
                                      int OC, int precision, void *stream) {
    if (precision != GPT2_FP32 && precision != GPT2_BF16) return fail(nullptr, GPT2_EINVAL, "unknown precision");
    PrecScope prec_scope(precision);
    KCK(linear_fwd(out, inp, W, bias, N, K, OC, EPI_STORE, nullptr, nullptr, (hipStream_t)stream));
    return GPT2_OK;
}

size_t gpt2k_linear_backward_work(int N, int K, int OC) {
    size_t a = 0, b = 0;
    bwd_split_need(N, K, OC, true, a, b);
    return align_up(a) + align_up(b) + align_up((size_t)16 * OC);
}

gpt2_status gpt2k_linear_backward(float *dinp, float *dW, float *dbias, const float *dout, const float *inp,
                                  const float *W, int N, int K, int OC, float *work, void *stream) {
    return gpt2k_linear_backward_prec(dinp, dW, dbias, dout, inp, W, N, K, OC, work, GPT2_FP32, stream);
}

gpt2_status gpt2k_linear_backward_prec(float *dinp, float *dW, float *dbias, const float *dout, const float *inp,
                                       const float *W, int N, int K, int OC, float *work, int precision,
                                       void *stream) {
    if (precision != GPT2_FP32 && precision != GPT2_BF16) return fail(nullptr, GPT2_EINVAL, "unknown precision");
    PrecScope prec_scope(precision);
    hipStream_t s = (hipStream_t)stream;
    size_t a = 0, b = 0;
    bwd_split_need(N, K, OC, true, a, b);
    float *splitk = work, *splitk_dw = work + align_up(a), *dbias_ws = splitk_dw + align_up(b);
    KCK(linear_bwd(dinp, EPI_STORE, nullptr, dW, dbias, dout, inp, W, N, K, OC, splitk, splitk_dw, dbias_ws, s));
    return GPT2_OK;
}

gpt2_status gpt2k_layernorm_forward(float *out, float *mean, float *rstd, const float *inp, const float *w,
                                    const float *b, int N, int C, void *stream) {
    KCK(k_layernorm_forward(out, mean, rstd, inp, w, b, N, C, (hipStream_t)stream));
    return GPT2_OK;
}

size_t gpt2k_layernorm_backward_work(int N, int C) { return (size_t)ln_partials(N) * 2 * C; }

gpt2_status gpt2k_layernorm_backward(float *dinp, float *dw, float *db, const float *dout, const float *inp,
                                     const float *w, const float *mean, const float *rstd, int N, int C,
                                     int accumulate, float *work, void *stream) {
    KCK(k_layernorm_backward(dinp, dw, db, work, dout, inp, w, mean, rstd, N, C, accumulate != 0,
                             (hipStream_t)stream));
    return GPT2_OK;
}

static bool attn_shape_ok(int B, int T, int C, int NH) {
    return B > 0 && T > 0 && T <= 1024 && T % 4 == 0 && NH > 0 && C % NH == 0 && (C / NH) % 4 == 0;
}
// the fused kernels take any T (their T x T workspace rows are padded to a multiple of 4)
static bool flash_shape_ok(int B, int T, int C, int NH) {
    return B > 0 && T > 0 && T <= 1024 && NH > 0 && C % NH == 0 && flash_attention_supported(C / NH);
}

gpt2_status gpt2k_attention_forward(float *atty, float *att, const float *qkv, int B, int T, int C, int NH,
                                    void *stream) {
    if (!attn_shape_ok(B, T, C, NH)) return fail(nullptr, GPT2_EINVAL, "attention shape not supported");
    KCK(attention_fwd(atty, att, qkv, B, T, C, NH, (hipStream_t)stream));
    return GPT2_OK;
}

size_t gpt2k_attention_backward_work(int B, int T, int C, int NH) {
    (void)C;
    return (size_t)B * NH * T * T;
}

gpt2_status gpt2k_attention_backward(float *dqkv, const float *datty, const float *qkv, const float *att, int B,
                                     int T, int C, int NH, float *work, void *stream) {
    if (!attn_shape_ok(B, T, C, NH)) return fail(nullptr, GPT2_EINVAL, "attention shape not supported");
    KCK(attention_bwd(dqkv, work, datty, qkv, att, B, T, C, NH, (hipStream_t)stream));
    return GPT2_OK;
}

size_t gpt2k_flash_attention_work(int B, int T, int C, int NH) {
    if (B <= 0 || T <= 0 || NH <= 0 || C % NH) return 0;
    return align_up((size_t)B * NH * T) + flash_attention_work(B, T, C, NH);
}

gpt2_status gpt2k_flash_attention_forward(float *atty, float *lse, const float *qkv, int B, int T, int C, int NH,
                                          float *work, void *stream) {
    if (!flash_shape_ok(B, T, C, NH))
        return fail(nullptr, GPT2_EINVAL, "fused attention supports head dims 16, 32, 64 and T <= 1024");
    KCK(flash_attention_forward(atty, lse, work + align_up((size_t)B * NH * T), qkv, B, T, C, NH,
                                (hipStream_t)stream));
    return GPT2_OK;
}

gpt2_status gpt2k_flash_attention_backward(float *dqkv, const float *datty, const float *qkv, const float *atty,
                                           const float *lse, int B, int T, int C, int NH, float *work,
                                           void *stream) {
    if (!flash_shape_ok(B, T, C, NH))
        return fail(nullptr, GPT2_EINVAL, "fused attention supports head dims 16, 32, 64 and T <= 1024");
    float *Dbuf = work, *ws = work + align_up((size_t)B * NH * T);
    KCK(flash_backward(dqkv, Dbuf, ws, datty, qkv, atty, lse, B, T, C, NH, (hipStream_t)stream));
    return GPT2_OK;
}

gpt2_status gpt2k_gelu_forward(float *out, const float *inp, size_t n, void *stream) {
    KCK(k_gelu_forward(out, inp, n, (hipStream_t)stream));
    return GPT2_OK;
}

gpt2_status gpt2k_gelu_backward(float *dinp, const float *inp, const float *dout, size_t n, void *stream) {
    KCK(k_gelu_backward(dinp, inp, dout, n, (hipStream_t)stream));
    return GPT2_OK;
}

gpt2_status gpt2k_crossentropy(float *logits, float *losses, float *loss, const int32_t *targets, int BT, int V,
                               int Vp, void *stream) {
    if (V <= 0 || Vp < V || BT <= 0) return fail(nullptr, GPT2_EINVAL, "bad crossentropy shape");
    KCK(k_crossentropy(logits, losses, targets, BT, V, Vp, 1.0f / BT, nullptr, (hipStream_t)stream));
    KCK(k_mean(loss, losses, BT, (hipStream_t)stream));
    return GPT2_OK;
}

gpt2_status gpt2k_encoder_forward(float *out, const int32_t *ids, const float *wte, const float *wpe, int B, int T,
                                  int C, int V, void *stream) {
    if (C % 4) return fail(nullptr, GPT2_EINVAL, "C must be a multiple of 4");
    KCK(k_encoder_forward(out, ids, wte, wpe, B, T, C, V, (hipStream_t)stream));
    return GPT2_OK;
}

size_t gpt2k_token_order_work(int BT) { return BT > 0 ? k_token_prep_work(BT) : 0; }

gpt2_status gpt2k_token_order(int32_t *order, int32_t *err_flag, const int32_t *ids, const int32_t *targets,
                              int BT, int V, int32_t *work, void *stream) {
    if (BT <= 0 || V <= 0) return fail(nullptr, GPT2_EINVAL, "BT and V must be positive");
    if (k_token_prep_work(BT) && !work) return fail(nullptr, GPT2_EINVAL, "work is required at this BT");
    KCK(k_token_prep(ids, targets, order, err_flag, work, BT, V, (hipStream_t)stream));
    return GPT2_OK;
}

size_t gpt2k_encoder_backward_work(int B, int T, int C) { return (size_t)B * T * C; }

gpt2_status gpt2k_encoder_backward(float *dwte, float *dwpe, const float *dout, const int32_t *ids,
                                   const int32_t *order, int B, int T, int C, int V, float *work, void *stream) {
    if (C % 4) return fail(nullptr, GPT2_EINVAL, "C must be a multiple of 4");
    KCK(k_encoder_backward(dwte, dwpe, work, dout, ids, order, B, T, C, V, (hipStream_t)stream));
    return GPT2_OK;
}

gpt2_status gpt2k_adamw(float *params, const float *grads, float *m, float *v, size_t n, float lr, float beta1,
                        float beta2, float eps, float weight_decay, int t, void *stream) {
    if (t < 1) return fail(nullptr, GPT2_EINVAL, "t must be >= 1");
    double c1 = 1.0 - std::pow((double)beta1, t), c2 = 1.0 - std::pow((double)beta2, t);
    KCK(k_adamw(params, grads, m, v, n, lr, beta1, beta2, eps, weight_decay, (float)c1, (float)c2, nullptr,
                (hipStream_t)stream));
    return GPT2_OK;
}

gpt2_status gpt2k_probe_mfma(float *out, int iters, double *flops, void *stream) {
    KCK(probe_mfma(out, iters, (hipStream_t)stream, flops));
    return GPT2_OK;
}

gpt2_status gpt2k_probe_copy(float *dst, const float *src, size_t n, void *stream) {
    KCK(probe_copy(dst, src, n, (hipStream_t)stream));
    return GPT2_OK;
}

}  // extern "C"

// ====================================================================== launch audit replay

namespace {

// Named element ranges of the caller's buffers (disjoint), and the check of
// every declared access against them: an access must stay inside the range
// it starts in, cover a run of adjacent ranges exactly (a launch over a whole
// stacked tensor or a whole parameter buffer), or cover one whole caller
// buffer exactly (a clear of it at build time).
class LayoutChecker : public AuditSink {
   public:
    struct Region {
        uintptr_t lo, hi;
        std::string name;
    };
    std::vector<Region> regs;
    std::vector<std::pair<uintptr_t, uintptr_t>> buffers;  // whole caller buffers
    long long nranges = 0;
    std::vector<std::string> violations;

    void add(uintptr_t base, size_t first, size_t count, int parts, const std::string &name) {
        if (!count) return;
        const size_t each = count / (size_t)parts;
        for (int p = 0; p < parts; p++) {
            const size_t c = p + 1 < parts ? each : count - each * (parts - 1);
            const uintptr_t lo = base + (first + (size_t)p * each) * 4;
            regs.push_back(Region{lo, lo + c * 4, parts > 1 ? name + "[" + std::to_string(p) + "]" : name});
        }
    }
    void seal() {
        std::sort(regs.begin(), regs.end(), [](const Region &a, const Region &b) { return a.lo < b.lo; });
    }
    void shrink(const std::string &name, size_t floats) {
        for (Region &r : regs)
            if (r.name == name) r.hi -= std::min<uintptr_t>(r.hi - r.lo, floats * 4);
    }
    void range(const char *kernel, const char *operand, const void *p, size_t bytes, bool write) override {
        nranges++;
        const uintptr_t lo = (uintptr_t)p, hi = lo + bytes;
        for (const auto &b : buffers)
            if (lo == b.first && hi == b.second) return;
        auto it = std::upper_bound(regs.begin(), regs.end(), lo,
                                   [](uintptr_t x, const Region &r) { return x < r.lo; });
        std::string what;
        if (it == regs.begin() || lo >= (it - 1)->hi) {
            what = "starts outside every tensor";
        } else {
            auto r = it - 1;
            if (hi <= r->hi) return;
            if (lo == r->lo) {  // a run of whole adjacent ranges?
                auto q = r;
                while (q->hi < hi && q + 1 != regs.end() && (q + 1)->lo == q->hi) ++q;
                if (q->hi == hi) return;
            }
            what = "runs past the end of " + r->name + " by " + std::to_string((long long)(hi - r->hi)) + " bytes";
        }
        if (violations.size() < 64)
            violations.push_back(std::string(kernel) + " " + operand + (write ? " (write)" : " (read)") + ": " + what);
        else if (violations.size() == 64)
            violations.push_back("...");
    }
};

}  // namespace

extern "C" {

gpt2_status gpt2_audit_step(const gpt2_config *cfg, int B, int T, const char *shrink_region, size_t shrink_floats,
                            char *report, size_t report_len, long long *n_ranges, long long *n_violations) {
    std::string why;
    if (!config_ok(cfg, B, T, &why)) return fail(nullptr, GPT2_EINVAL, why);
    if (audit_sink()) return fail(nullptr, GPT2_ESTATE, "a launch audit is already running on this thread");
    Layout l;
    make_layout(cfg, B, T, &l);
    // stand-in base addresses, far apart; never dereferenced
    auto base = [](int b) { return (uintptr_t)(b + 1) << 40; };
    LayoutChecker ck;
    static const char *bufnames[4] = {"params:", "grads:", "adam_m:", "adam_v:"};
    for (int b = 0; b < 4; b++)
        for (int i = 0; i < 16; i++)
            ck.add(base(b), l.poff[i], l.pcnt[i], (i >= 2 && i <= 13) ? l.L : 1, std::string(bufnames[b]) + kParamNames[i]);
    static const bool per_layer[NUM_ACTS] = {false, true, true, true, true, true, true, true, true, true, true,
                                             true,  true, true, false, false, false, false, false, false, true};
    for (int i = 0; i < NUM_ACTS; i++)
        ck.add(base(4), l.aoff[i], l.acnt[i], per_layer[i] ? l.L : 1, std::string("acts:") + kActNames[i]);
    for (int i = 0; i < l.nwreg; i++)
        ck.add(base(5), l.wreg[i].off, l.wreg[i].cnt, l.wreg[i].parts, std::string("work:") + l.wreg[i].name);
    ck.add(base(6), l.i_tok, (size_t)l.BT, 1, "iwork:ids");
    ck.add(base(6), l.i_order, (size_t)l.BT, 1, "iwork:order");
    if (k_token_prep_work((int)l.BT)) ck.add(base(6), l.i_sort, k_token_prep_work((int)l.BT), 1, "iwork:sort");
    ck.add(base(6), l.i_err, 1, 1, "iwork:err");
    ck.add(base(6), l.i_dec, 1, 1, "iwork:decode_pos");
    ck.add(base(7), 0, (size_t)l.BT, 1, "caller:inputs");
    ck.add(base(8), 0, (size_t)l.BT, 1, "caller:targets");
    ck.add(base(9), 0, (size_t)l.B, 1, "caller:decode_tokens");
    ck.add(base(10), 0, (size_t)l.B, 1, "caller:coins");
    ck.add(base(11), 0, (size_t)l.B, 1, "caller:next");
    const size_t buf_floats[7] = {l.nparams, l.nparams, l.nparams, l.nparams, l.nacts, l.nwork, l.niwork};
    for (int b = 0; b < 7; b++) ck.buffers.push_back({base(b), base(b) + buf_floats[b] * 4});
    ck.seal();
    if (shrink_region && *shrink_region) ck.shrink(shrink_region, shrink_floats);

    gpt2_buffers dev{(float *)base(0), (float *)base(1), (float *)base(2), (float *)base(3),
                     (float *)base(4), (float *)base(5), (int32_t *)base(6)};
    set_audit_sink(&ck);
    gpt2_model *m = nullptr;
    gpt2_status st = gpt2_build(cfg, B, T, &dev, nullptr, nullptr, &m);
    const int32_t *inp = (const int32_t *)base(7), *tgt = (const int32_t *)base(8);
    if (st == GPT2_OK) st = gpt2_forward(m, inp, nullptr, nullptr);
    if (st == GPT2_OK) st = gpt2_forward(m, inp, tgt, nullptr);
    if (st == GPT2_OK) st = gpt2_zero_grad(m);
    if (st == GPT2_OK) st = gpt2_backward(m);
    if (st == GPT2_OK) st = gpt2_update(m, 1e-4f, 0.9f, 0.999f, 1e-8f, 0.0f, 1);
    const int32_t *dtok = (const int32_t *)base(9);
    const float *coins = (const float *)base(10);
    int32_t *dnext = (int32_t *)base(11);
    for (int pos : {0, T / 2, T - 1})
        if (st == GPT2_OK) st = gpt2_decode_step(m, dtok, pos, pos == 0 ? nullptr : coins, dnext);
    // and a step with bfloat16 products
    if (st == GPT2_OK) st = gpt2_set_matmul_precision(m, GPT2_BF16);
    if (st == GPT2_OK) st = gpt2_forward(m, inp, tgt, nullptr);
    if (st == GPT2_OK) st = gpt2_backward(m);
    set_audit_sink(nullptr);
    const std::string err = m ? m->err : g_last_error;
    gpt2_free(m);
    if (st != GPT2_OK) return fail(nullptr, st, "replay stopped: " + err);
    if (n_ranges) *n_ranges = ck.nranges;
    if (n_violations) *n_violations = (long long)ck.violations.size();
    if (report && report_len) {
        std::string txt;
        for (const std::string &v : ck.violations) txt += v + "\n";
        snprintf(report, report_len, "%s", txt.c_str());
    }
    return GPT2_OK;
}

}  // extern "C"
