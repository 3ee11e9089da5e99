/*
 * gpt2.h -- C ABI of libgpt2mi: one fp32 GPT-2 training step (forward,
 * backward, AdamW) on one AMD Instinct MI355X (gfx950), over flat 1-D device
 * buffers with fixed offsets.
 *
 * What the step computes is described on these pages:
 *  - "OpenAI創始大神手搓千行C代碼訓練GPT，附PyTorch遷移教程" (QbitAI), section
 *    "手動實現每個層前向/反向傳播": memory is allocated once as one 1-D array
 *    that every weight and activation points into; the footprint stays
 *    constant while batches flow through; each layer has a hand-written
 *    forward and backward, chained into one forward/backward/update loop.
 *  - "“真男人就應該用 C 編程”！用 1000 行 C 代碼手搓了一個大模型…" (InfoQ): the
 *    layer list (encoder, layernorm, matmul, self-attention, gelu, residual,
 *    softmax, cross-entropy), fp32 throughout, int32 token streams, Adam at
 *    lr 1e-4, and the GPT-2 124M header (1024 / 50257 / 12 / 12 / 768,
 *    124439808 parameters).
 *  - "Bản sao ChatGPT dựa trên GPT-2 được triển khai bằng 3000 byte C (2023)"
 *    (GeekNews), sections "Triển khai các lớp mạng nơ-ron" and
 *    "Phần lõi Transformer": the layer definitions and the block dataflow,
 *    including the tied token-embedding head.
 *
 * Conventions for every call:
 *  - Device memory is owned by the caller (allocated once, e.g. through
 *    PyTorch) and borrowed by the library for the handle's lifetime.  The
 *    library never allocates or frees device memory.
 *  - All work is enqueued, in order, on the HIP stream given to gpt2_build;
 *    calls return before the work finishes unless stated otherwise.
 *  - Calls return a gpt2_status; on failure gpt2_last_error(model) holds a
 *    message.  Nothing is printed, no exception crosses the ABI, and the
 *    process is never exited.
 *  - All floating-point data is IEEE fp32, row-major; tokens are int32.
 */
#ifndef GPT2_MI_H
#define GPT2_MI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GPT2_OK = 0,
    GPT2_EINVAL = -1,  /* bad argument, shape or configuration                 */
    GPT2_ERANGE = -2,  /* a token or target outside [0, vocab_size)            */
    GPT2_ESTATE = -3,  /* call out of order (e.g. backward before forward)     */
    GPT2_EDEVICE = -4, /* a HIP runtime call or kernel launch failed           */
    GPT2_EIO = -5      /* a file could not be read or written, or is damaged   */
} gpt2_status;

/* Model shape.  padded_vocab_size >= vocab_size is the row count of wte and
 * the column count of the logits (the extra rows/columns are zero and take
 * no part in the softmax).  channels % num_heads == 0; channels and the head
 * dimension must be multiples of 4; channels <= 2048. */
typedef struct {
    int max_seq_len;       /* rows of the position embedding wpe          */
    int vocab_size;        /* V                                            */
    int padded_vocab_size; /* Vp                                           */
    int num_layers;        /* L                                            */
    int num_heads;         /* NH                                           */
    int channels;          /* C                                            */
} gpt2_config;

/* Element counts of the caller-allocated buffers for one (config, B, T). */
typedef struct {
    size_t params;    /* floats; grads, adam_m and adam_v have the same count */
    size_t acts;      /* floats: saved forward activations and the logits     */
    size_t work;      /* floats: backward temporaries and reduction scratch   */
    size_t iwork;     /* int32s: token order and the error flag               */
} gpt2_sizes;

/* Device pointers (all 256-byte aligned) of the caller-allocated buffers. */
typedef struct {
    float *params;    /* [params] the 16 parameter tensors, see gpt2_layout   */
    float *grads;     /* [params] same offsets as params                      */
    float *adam_m;    /* [params] AdamW first moment                          */
    float *adam_v;    /* [params] AdamW second moment                         */
    float *acts;      /* [acts]                                               */
    float *work;      /* [work]                                               */
    int32_t *iwork;   /* [iwork]                                              */
} gpt2_buffers;

typedef struct gpt2_model gpt2_model; /* opaque handle */

/* Precision of the linear-layer products (gpt2_set_matmul_precision). */
enum { GPT2_FP32 = 0, GPT2_BF16 = 1 };

/* Which table gpt2_layout reads. */
enum { GPT2_PARAMS = 0, GPT2_ACTS = 1 };

/* Buffer sizes for (cfg, B, T): the constant footprint allocated once up
 * front (QbitAI llm.c article, "手動實現每個層前向/反向傳播": every tensor a fixed
 * offset into memory allocated at the start).  Host only; B >= 1,
 * 1 <= T <= min(max_seq_len, 1024), T a multiple of 4 unless the head
 * dimension is 16, 32 or 64. */
gpt2_status gpt2_query_sizes(const gpt2_config *cfg, int B, int T, gpt2_sizes *out);

/* Entry idx of a layout table (host only).  The tensor order is explicit (the
 * GeekNews page, "Nạp trọng số", on a flat fp32 weight file whose tensors
 * must be placed in a stated order).  GPT2_PARAMS has 16 entries, in this
 * order, each stacked over layers where it is per layer:
 *   wte[Vp][C] wpe[maxT][C] ln1w[L][C] ln1b[L][C] qkvw[L][3C][C] qkvb[L][3C]
 *   attprojw[L][C][C] attprojb[L][C] ln2w[L][C] ln2b[L][C] fcw[L][4C][C]
 *   fcb[L][4C] fcprojw[L][C][4C] fcprojb[L][C] lnfw[C] lnfb[C]
 * (weights are out x in: row o holds the input weights of output o; qkv rows
 * are q | k | v blocks of C, head h owning columns h*hd..h*hd+hd-1 of each.)
 * The tensors are packed with no gaps: params = their sum (124439808 for
 * GPT-2 124M with Vp = V).  GPT2_ACTS lists the named activation tensors in
 * the acts buffer (offsets are padded to 64 floats):
 *   encoded[BT][C]; per layer ln1[BT][C] ln1_mean[BT] ln1_rstd[BT]
 *   qkv[BT][3C] att[B][NH][T][T] atty[BT][C] residual2[BT][C] ln2[BT][C]
 *   ln2_mean[BT] ln2_rstd[BT] fch[BT][4C] fch_gelu[BT][4C] residual3[BT][C]
 *   (each stacked over layers); lnf[BT][C] lnf_mean[BT] lnf_rstd[BT]
 *   logits[BT][Vp] losses[BT] loss[1] lse[L][B][NH][T].
 * When the head dimension is 16, 32 or 64 attention runs fused: att has 0
 * elements and lse holds each query's log-sum-exp of its scaled scores.
 * Otherwise lse has 0 elements and att holds the softmax probabilities: row
 * t is meaningful for u <= t and zero for t < u < round_up(t+1, 128).  After a forward with targets,
 * logits holds d(mean loss)/d(logits) instead (columns >= V are zero).
 * Returns GPT2_EINVAL for idx out of range; *name, *offset, *count may be
 * NULL.  The returned name is a static string. */
gpt2_status gpt2_layout(const gpt2_config *cfg, int B, int T, int which, int idx,
                        const char **name, size_t *offset, size_t *count);

/* Create a handle over caller buffers for fixed (B, T) (the one allocation
 * made at the start, QbitAI llm.c article, "手動實現每個層前向/反向傳播").  If
 * init_params_host is non-NULL it is copied (params floats, host memory) into
 * dev->params; otherwise dev->params is left as is.  grads, adam_m and adam_v are set to
 * zero.  hip_stream is a hipStream_t (NULL = the null stream).  The buffers
 * must hold at least the counts of gpt2_query_sizes. */
gpt2_status gpt2_build(const gpt2_config *cfg, int B, int T, const gpt2_buffers *dev,
                       const float *init_params_host, void *hip_stream, gpt2_model **out);

/* Forward pass over one batch (the forward half of the loop in the QbitAI
 * llm.c article, "手動實現每個層前向/反向傳播"; the layer order of the GeekNews
 * page, "Phần lõi Transformer"; int32 token streams as in the InfoQ article's
 * walkthrough).  inputs and targets are DEVICE pointers to B*T int32 token
 * ids, row-major [B][T], already resident in HBM (targets may be NULL:
 * logits only); they are copied into the model's own buffer, so the caller
 * may reuse them once the call's work has run.  With targets, the
 * per-position losses, their mean, and d(mean loss)/d(logits) (in place of
 * the logits) are produced, which enables gpt2_backward.
 *
 * Ids are checked on the device, not on the host (no synchronization).  An id
 * outside [0, V) sets the model's error flag; for memory safety it is then
 * read as the nearest valid id.  While the flag is set the step changes no
 * trainable state: the loss gradient of every batch is written as zeros
 * (losses as NaN), so gpt2_backward adds exact zeros to grads, and
 * gpt2_update leaves params, adam_m and adam_v untouched.  The flag stays set
 * until a waiting call reports it: this call when mean_loss is non-NULL
 * (then it waits for the stream, stores the mean loss in the host float
 * *mean_loss and returns GPT2_ERANGE), or gpt2_sync.  After such a report the
 * batch may not be back-propagated (gpt2_backward returns GPT2_ESTATE until
 * the next forward with targets). */
gpt2_status gpt2_forward(gpt2_model *model, const int32_t *inputs, const int32_t *targets,
                         float *mean_loss);

/* grads = 0 over the whole parameter buffer (the gradients are accumulated
 * by gpt2_backward, so the caller clears them once per step). */
gpt2_status gpt2_zero_grad(gpt2_model *model);

/* Backward pass of the mean loss of the last forward-with-targets, layer by
 * layer in reverse (the hand-written backward of each layer in the QbitAI
 * llm.c article, "手動實現每個層前向/反向傳播"): grads += d(mean loss)/d(params).
 * GPT2_ESTATE without such a forward. */
gpt2_status gpt2_backward(gpt2_model *model);

/* The parameter update that closes the loop (Adam at lr 1e-4 in the InfoQ
 * article's walkthrough; AdamW with decoupled weight decay here, identical to
 * Adam at weight_decay 0), one pass over the flat buffers:
 * m = b1 m + (1-b1) g; v = b2 v + (1-b2) g^2;
 * theta -= lr (m/(1-b1^t) / (sqrt(v/(1-b2^t)) + eps) + weight_decay theta).
 * t is the 1-based step count (GPT2_EINVAL if t < 1).  Skipped on the device
 * while the error flag of gpt2_forward is set. */
gpt2_status gpt2_update(gpt2_model *model, float lr, float beta1, float beta2, float eps,
                        float weight_decay, int t);

/* One autoregressive decoding step with the key/value cache held in the
 * model's own activation buffer (the GeekNews page, "Cách KV caching hoạt
 * động": the keys and values of the tokens already processed are kept and
 * only the new token's row is computed; "Phép nhân ma trận nhanh": only the
 * new rows of each product are multiplied; the InfoQ article's run prints the
 * ids sampled after training).
 *
 * tokens: DEVICE int32[B], the token at position pos of each of the B
 * sequences (0 <= pos < T).  Rows (b, u < pos) of every layer's qkv
 * activations must hold the keys and values of the earlier positions: from
 * gpt2_forward over ids whose first pos positions are the prompt (a prefill;
 * the later positions are not read), or from earlier decode steps.  The call
 * computes row (b, pos) through every layer, writes its q | k | v into each
 * layer's qkv rows (extending the cache) and its logits into row (b, pos) of
 * the logits activation, and stores the next token of each sequence in
 * next (DEVICE int32[B]): the most probable token (lowest id among equal
 * maxima) when coins is NULL, otherwise, with p the softmax of the logits
 * over v < V, the first v whose cumulative probability exceeds coins[b]
 * (DEVICE float[B] of uniform draws in [0, 1) chosen by the caller).
 * Asynchronous; ids outside [0, V) raise the model's error flag (reported by
 * gpt2_sync) and are read as the nearest valid id.  Only activation rows
 * (b, pos) and the work buffer are written, so a following gpt2_backward needs
 * a new forward with targets (GPT2_ESTATE otherwise). */
gpt2_status gpt2_decode_step(gpt2_model *model, const int32_t *tokens, int pos, const float *coins, int32_t *next);

/* Precision of the linear-layer products of gpt2_forward and gpt2_backward
 * (the QbitAI llm.c article, "手動實現每個層前向/反向傳播", names fp16 and lower
 * precision as the trainer's next step).  GPT2_FP32 (the default): fp32
 * products.  GPT2_BF16: the operands of every linear-layer product -- qkv,
 * attention projection, MLP and the tied head, forward and backward -- are
 * rounded to bfloat16 (to nearest even) on their way to the matrix unit and
 * accumulated in fp32; everything stored stays fp32: parameters (the master
 * weights), gradients, AdamW moments and activations.  Attention, LayerNorm,
 * softmax, GELU, bias gradients and AdamW are fp32 in both modes.  Takes
 * effect for the calls enqueued after it; GPT2_EINVAL for other values. */
gpt2_status gpt2_set_matmul_precision(gpt2_model *model, int precision);

/* Wait for the stream; GPT2_ERANGE if an out-of-range id was seen since the
 * last report (the flag is then cleared, and gpt2_backward needs a new
 * forward with targets), GPT2_EDEVICE on a HIP error. */
gpt2_status gpt2_sync(gpt2_model *model);

/* Per-launch timing of the step (tracing).  While enabled, every kernel
 * launch made by gpt2_forward / gpt2_zero_grad / gpt2_backward / gpt2_update
 * is bracketed by two HIP events on the model's stream.  gpt2_profile_read
 * waits for the stream, then returns one entry per kernel name (the name a
 * kernel-trace profiler shows) with the number of launches, the summed
 * event-to-event time, and the summed algorithmic FLOPs and bytes (the
 * compulsory operand traffic of each launch; causal products count only the
 * u <= t triangle); it then clears the records.  *n_entries gets the number
 * of names; at most max_entries are written.  Enabling creates HIP events
 * (host-side runtime objects); nothing is allocated during a step. */
typedef struct {
    char name[128];
    long long launches;
    double ms;
    double flops;
    double bytes;
} gpt2_profile_entry;
gpt2_status gpt2_profile_enable(gpt2_model *model, int enable);
gpt2_status gpt2_profile_read(gpt2_model *model, gpt2_profile_entry *out, int max_entries, int *n_entries);

/* Checkpoints of the training state (the femtoGPT page, "使用方法": training
 * may stop and resume at any time from its saved state; the GeekNews page,
 * "Nạp trọng số": a flat fp32 weight file, read in an explicitly stated
 * tensor order).  The file holds a header (magic, version, the six config
 * fields, the step count t, the 16-entry parameter table of gpt2_layout with
 * names, offsets and counts, and a 64-bit checksum of the payload) followed
 * by params, adam_m and adam_v as raw little-endian fp32, in that order.
 * Gradients and activations are not saved (gradients are cleared every
 * step).  Both calls wait for the model's stream and copy through a 16 MiB
 * host staging buffer; no device memory is allocated.
 *
 * gpt2_save_checkpoint writes `path` (through `path`.tmp, renamed when
 * complete, so a failed save leaves any older file in place).  t >= 0 is the
 * number of optimizer steps taken (the next gpt2_update passes t + 1).
 * gpt2_load_checkpoint reads a file written for the same config (any B, T),
 * verifies its header, size and checksum before copying anything, then
 * overwrites params, adam_m and adam_v and stores the saved step count in
 * *t (may be NULL).  A mismatched config or tensor table is GPT2_EINVAL, an
 * unreadable, truncated or corrupted file GPT2_EIO; in both cases the model
 * is unchanged.  After a load, gpt2_backward needs a new forward. */
gpt2_status gpt2_save_checkpoint(gpt2_model *model, const char *path, int t);
gpt2_status gpt2_load_checkpoint(gpt2_model *model, const char *path, int *t);

/* Release the handle (not the caller's buffers). */
void gpt2_free(gpt2_model *model);

/* Message of the last failure on this handle ("" if none); with a NULL
 * handle, of the last failure of a call that had no handle to report on. */
const char *gpt2_last_error(const gpt2_model *model);

#ifdef __cplusplus
}
#endif
#endif /* GPT2_MI_H */
