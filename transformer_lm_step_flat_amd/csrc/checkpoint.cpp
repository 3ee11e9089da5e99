// Checkpoint file format (see checkpoint.h): header, parameter table,
// checksum, then params, adam_m and adam_v as raw fp32.
#include "checkpoint.h"

#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

namespace {

constexpr char kMagic[8] = {'G', 'P', 'T', '2', 'M', 'I', 'c', 'k'};
constexpr uint32_t kVersion = 1;
constexpr uint64_t kFnvOffset = 14695981039346656037ULL, kFnvPrime = 1099511628211ULL;

struct Tensor {
    char name[16];
    int64_t offset, count;
};
struct Header {
    char magic[8];
    uint32_t version, header_bytes;
    int32_t cfg[6];
    int32_t t, ntensors;
    int64_t nparams;
    Tensor tensors[16];
    uint64_t checksum;
};
static_assert(sizeof(Header) == kCkHeaderBytes, "checkpoint header layout");

// FNV-1a over the 8-byte words of n floats (n even)
void fnv_words(uint64_t &h, const float *p, size_t n) {
    for (size_t i = 0; i < n / 2; i++) {
        uint64_t w;
        memcpy(&w, p + 2 * i, 8);
        h ^= w;
        h *= kFnvPrime;
    }
}

Header header_for(const CkModel &m, int t) {
    Header h;
    memset(&h, 0, sizeof h);
    memcpy(h.magic, kMagic, 8);
    h.version = kVersion;
    h.header_bytes = (uint32_t)kCkHeaderBytes;
    memcpy(h.cfg, m.cfg, sizeof h.cfg);
    h.t = t;
    h.ntensors = 16;
    h.nparams = m.nparams;
    for (int i = 0; i < 16; i++) {
        strncpy(h.tensors[i].name, m.names[i], sizeof h.tensors[i].name - 1);
        h.tensors[i].offset = m.offset[i];
        h.tensors[i].count = m.count[i];
    }
    h.checksum = kFnvOffset;
    return h;
}

int fail(std::string *err, int code, const std::string &msg) {
    if (err) *err = msg;
    return code;
}

}  // namespace

int ck_save(const char *path, const CkModel &m, int t, const CkFetch &fetch, std::string *err) {
    if (!path || !*path) return fail(err, CK_EINVAL, "path is empty");
    if (t < 0) return fail(err, CK_EINVAL, "t must be >= 0");
    if (m.nparams <= 0 || m.nparams % 2) return fail(err, CK_EINVAL, "parameter count must be positive and even");
    const size_t n = (size_t)m.nparams;
    Header h = header_for(m, t);
    const std::string tmp = std::string(path) + ".tmp";
    FILE *f = fopen(tmp.c_str(), "wb");
    if (!f) return fail(err, CK_EIO, "cannot open " + tmp + " for writing");
    std::vector<float> buf(std::min(n, kCkChunkFloats));
    bool ok = fwrite(&h, sizeof h, 1, f) == 1;
    bool copied = true;
    uint64_t sum = h.checksum;
    for (int a = 0; a < 3 && ok && copied; a++)
        for (size_t i = 0; i < n && ok && copied; i += buf.size()) {
            const size_t k = std::min(buf.size(), n - i);
            copied = fetch(a, i, k, buf.data()) == 0;
            if (!copied) break;
            fnv_words(sum, buf.data(), k);
            ok = fwrite(buf.data(), sizeof(float), k, f) == k;
        }
    h.checksum = sum;
    if (ok && copied) ok = fseek(f, 0, SEEK_SET) == 0 && fwrite(&h, sizeof h, 1, f) == 1;
    ok = (fclose(f) == 0) && ok;
    if (!copied) {
        remove(tmp.c_str());
        return fail(err, CK_ECOPY, "copy from the device failed");
    }
    if (!ok || rename(tmp.c_str(), path) != 0) {
        remove(tmp.c_str());
        return fail(err, CK_EIO, std::string("cannot write ") + path);
    }
    return CK_OK;
}

int ck_load(const char *path, const CkModel &m, int *t, const CkStore &store, std::string *err) {
    if (!path || !*path) return fail(err, CK_EINVAL, "path is empty");
    if (m.nparams <= 0 || m.nparams % 2) return fail(err, CK_EINVAL, "parameter count must be positive and even");
    const size_t n = (size_t)m.nparams;
    FILE *f = fopen(path, "rb");
    if (!f) return fail(err, CK_EIO, std::string("cannot open ") + path);
    auto bad = [&](int code, const std::string &msg) {
        fclose(f);
        return fail(err, code, std::string(path) + ": " + msg);
    };
    Header h;
    if (fread(&h, sizeof h, 1, f) != 1) return bad(CK_EIO, "shorter than a checkpoint header");
    if (memcmp(h.magic, kMagic, 8) != 0) return bad(CK_EIO, "not a checkpoint of this library");
    if (h.version != kVersion || h.header_bytes != kCkHeaderBytes) return bad(CK_EIO, "unknown checkpoint version");
    const Header want = header_for(m, h.t);
    if (memcmp(h.cfg, want.cfg, sizeof h.cfg) != 0) return bad(CK_EINVAL, "saved for another model configuration");
    if (h.ntensors != 16 || h.nparams != want.nparams) return bad(CK_EINVAL, "parameter count differs");
    for (int i = 0; i < 16; i++)
        if (strncmp(h.tensors[i].name, want.tensors[i].name, sizeof h.tensors[i].name) != 0 ||
            h.tensors[i].offset != want.tensors[i].offset || h.tensors[i].count != want.tensors[i].count)
            return bad(CK_EINVAL, std::string("tensor table differs at ") + want.tensors[i].name);
    if (h.t < 0) return bad(CK_EIO, "negative step count");
    if (fseek(f, 0, SEEK_END) != 0) return bad(CK_EIO, "cannot seek");
    const long long size = ftell(f);
    if (size != (long long)(kCkHeaderBytes + 3 * n * sizeof(float))) return bad(CK_EIO, "truncated or oversized");
    // verify the whole payload before any of it is stored
    std::vector<float> buf(std::min(n, kCkChunkFloats));
    uint64_t sum = kFnvOffset;
    if (fseek(f, (long)kCkHeaderBytes, SEEK_SET) != 0) return bad(CK_EIO, "cannot seek");
    for (int a = 0; a < 3; a++)
        for (size_t i = 0; i < n; i += buf.size()) {
            const size_t k = std::min(buf.size(), n - i);
            if (fread(buf.data(), sizeof(float), k, f) != k) return bad(CK_EIO, "read failed");
            fnv_words(sum, buf.data(), k);
        }
    if (sum != h.checksum) return bad(CK_EIO, "checksum mismatch (the file is damaged)");
    if (fseek(f, (long)kCkHeaderBytes, SEEK_SET) != 0) return bad(CK_EIO, "cannot seek");
    for (int a = 0; a < 3; a++)
        for (size_t i = 0; i < n; i += buf.size()) {
            const size_t k = std::min(buf.size(), n - i);
            if (fread(buf.data(), sizeof(float), k, f) != k) return bad(CK_EIO, "read failed");
            if (store(a, i, k, buf.data()) != 0) return bad(CK_ECOPY, "copy to the device failed");
        }
    fclose(f);
    if (t) *t = h.t;
    return CK_OK;
}
