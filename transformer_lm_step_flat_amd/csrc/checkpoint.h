// Checkpoint files of the training state: host-only C++ (no HIP), so that
// the format code can be built and checked on its own.  The device copies
// are callbacks supplied by the caller.
//
// A checkpoint holds what training needs to continue: the step count t, the
// parameters and AdamW's two moments (the femtoGPT page, "使用方法": training
// can stop and resume at any time from its saved state; the GeekNews page,
// "Nạp trọng số": a flat fp32 weight file is only usable with its tensor
// order stated, so the order is written into the file).  Little-endian:
//   0   char[8]   magic "GPT2MIck"
//   8   uint32    version (1)
//   12  uint32    header bytes (576)
//   16  int32[6]  max_seq_len, vocab_size, padded_vocab_size, num_layers, num_heads, channels
//   40  int32     t (optimizer steps taken)
//   44  int32     tensor count (16)
//   48  int64     floats per array (the parameter count n, even)
//   56  16 x {char name[16]; int64 offset; int64 count}   the parameter table
//   568 uint64    FNV-1a 64 of the payload, taken over its 8-byte words
//   576 float32   params[n], adam_m[n], adam_v[n]
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <functional>
#include <string>

struct CkModel {
    int32_t cfg[6];
    int64_t nparams;
    const char *names[16];
    int64_t offset[16], count[16];
};

enum { CK_OK = 0, CK_EINVAL = 1, CK_EIO = 2, CK_ECOPY = 3 };

constexpr size_t kCkHeaderBytes = 576;
constexpr size_t kCkChunkFloats = (size_t)1 << 22;  // staged per copy (16 MiB)

// fetch(array, first, count, dst): copy `count` floats of array 0 (params),
// 1 (adam_m) or 2 (adam_v) from element `first` into host dst; 0 on success.
using CkFetch = std::function<int(int, size_t, size_t, float *)>;
// store(array, first, count, src): the reverse; 0 on success.
using CkStore = std::function<int(int, size_t, size_t, const float *)>;

// Write `path` through `path`.tmp, renamed when complete.
int ck_save(const char *path, const CkModel &m, int t, const CkFetch &fetch, std::string *err);
// Verify header, size and checksum of `path` against m, then store the three
// arrays (nothing is stored unless the whole file checks out); *t gets the
// saved step count.
int ck_load(const char *path, const CkModel &m, int *t, const CkStore &store, std::string *err);
