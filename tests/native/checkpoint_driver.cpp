// Host-only check of the checkpoint file code (csrc/checkpoint.cpp), built
// with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_native_sanitized.py.  "Device" arrays are host vectors here.
// Exit status 0 when every check holds; a sanitizer report aborts.
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "../../transformer_lm_step_flat_amd/csrc/checkpoint.h"

static int failures = 0;
#define CHECK(c)                                                   \
    do {                                                           \
        if (!(c)) {                                                \
            fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            failures++;                                            \
        }                                                          \
    } while (0)

static const char *kNames[16] = {"wte", "wpe", "ln1w", "ln1b", "qkvw", "qkvb", "attprojw", "attprojb",
                                 "ln2w", "ln2b", "fcw", "fcb", "fcprojw", "fcprojb", "lnfw", "lnfb"};

static CkModel model(int64_t n, int L) {
    CkModel m;
    const int32_t cfg[6] = {64, 65, 128, L, 4, 64};
    memcpy(m.cfg, cfg, sizeof cfg);
    m.nparams = n;
    int64_t off = 0;
    for (int i = 0; i < 16; i++) {
        m.names[i] = kNames[i];
        m.count[i] = n / 16 + (i == 15 ? n % 16 : 0);
        m.offset[i] = off;
        off += m.count[i];
    }
    return m;
}

static std::vector<unsigned char> slurp(const std::string &p) {
    std::vector<unsigned char> b;
    FILE *f = fopen(p.c_str(), "rb");
    if (!f) return b;
    int c;
    while ((c = fgetc(f)) != EOF) b.push_back((unsigned char)c);
    fclose(f);
    return b;
}
static void spit(const std::string &p, const std::vector<unsigned char> &b) {
    FILE *f = fopen(p.c_str(), "wb");
    if (!f) return;
    fwrite(b.data(), 1, b.size(), f);
    fclose(f);
}

static void round_trip(const std::string &dir, int64_t n) {
    const CkModel m = model(n, 2);
    std::vector<float> src[3], dst[3];
    for (int a = 0; a < 3; a++) {
        src[a].resize(n);
        dst[a].assign(n, -7.0f);
        for (int64_t i = 0; i < n; i++) src[a][i] = (float)((i * 2654435761u + a * 97u) % 100003) * 1e-3f - 50.0f;
    }
    auto fetch = [&](int a, size_t first, size_t count, float *out) {
        if (a < 0 || a > 2 || first + count > (size_t)n) return 1;
        memcpy(out, src[a].data() + first, count * sizeof(float));
        return 0;
    };
    auto store = [&](int a, size_t first, size_t count, const float *in) {
        if (a < 0 || a > 2 || first + count > (size_t)n) return 1;
        memcpy(dst[a].data() + first, in, count * sizeof(float));
        return 0;
    };
    const std::string path = dir + "/rt_" + std::to_string(n) + ".ck";
    std::string err;
    CHECK(ck_save(path.c_str(), m, 42, fetch, &err) == CK_OK);
    const std::vector<unsigned char> file = slurp(path);
    CHECK(file.size() == kCkHeaderBytes + 3 * (size_t)n * 4);
    int t = -1;
    CHECK(ck_load(path.c_str(), m, &t, store, &err) == CK_OK);
    CHECK(t == 42);
    for (int a = 0; a < 3; a++) CHECK(memcmp(src[a].data(), dst[a].data(), n * sizeof(float)) == 0);

    // damaged files are refused before anything is stored
    for (int a = 0; a < 3; a++) dst[a].assign(n, -7.0f);
    auto untouched = [&]() {
        for (int a = 0; a < 3; a++)
            for (int64_t i = 0; i < n; i++)
                if (dst[a][i] != -7.0f) return false;
        return true;
    };
    std::vector<unsigned char> bad = file;
    bad[kCkHeaderBytes + bad.size() / 2 - kCkHeaderBytes / 2] ^= 0x10;
    spit(dir + "/flip.ck", bad);
    CHECK(ck_load((dir + "/flip.ck").c_str(), m, &t, store, &err) == CK_EIO);
    bad = file;
    bad.pop_back();
    spit(dir + "/short.ck", bad);
    CHECK(ck_load((dir + "/short.ck").c_str(), m, &t, store, &err) == CK_EIO);
    bad.assign(file.begin(), file.begin() + 100);
    spit(dir + "/header.ck", bad);
    CHECK(ck_load((dir + "/header.ck").c_str(), m, &t, store, &err) == CK_EIO);
    bad = file;
    bad[0] = 'X';
    spit(dir + "/magic.ck", bad);
    CHECK(ck_load((dir + "/magic.ck").c_str(), m, &t, store, &err) == CK_EIO);
    // another configuration, another tensor table
    const CkModel other = model(n, 3);
    CHECK(ck_load(path.c_str(), other, &t, store, &err) == CK_EINVAL);
    CkModel shifted = m;
    shifted.offset[3] += 2;
    shifted.count[3] -= 2;
    shifted.count[2] += 2;
    CHECK(ck_load(path.c_str(), shifted, &t, store, &err) == CK_EINVAL);
    CHECK(ck_load((dir + "/missing.ck").c_str(), m, &t, store, &err) == CK_EIO);
    CHECK(untouched());
    // a failing device copy is reported as such
    auto broken = [&](int, size_t, size_t, const float *) { return 1; };
    CHECK(ck_load(path.c_str(), m, &t, broken, &err) == CK_ECOPY);
    auto broken_fetch = [&](int, size_t, size_t, float *) { return 1; };
    CHECK(ck_save((dir + "/nofetch.ck").c_str(), m, 1, broken_fetch, &err) == CK_ECOPY);
    CHECK(slurp(dir + "/nofetch.ck").empty());
    CHECK(ck_save(path.c_str(), m, -1, fetch, &err) == CK_EINVAL);
    const CkModel odd = model(n + 1, 2);
    CHECK(ck_save((dir + "/odd.ck").c_str(), odd, 1, fetch, &err) == CK_EINVAL);
}

int main(int argc, char **argv) {
    if (argc < 2) return 2;
    const std::string dir = argv[1];
    round_trip(dir, 1024);                        // one chunk
    round_trip(dir, (int64_t)kCkChunkFloats + 4096);  // two chunks per array, the last one short
    round_trip(dir, 3 * (int64_t)kCkChunkFloats / 2 + 2);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("checkpoint driver: all checks passed\n");
    return 0;
}
