// Launch audit (host only).  While a sink is installed on the calling thread,
// every launcher of the library declares the element ranges its kernels
// would read or write, computed from the kernels' index formulas, grid and
// leading dimensions, and returns without launching anything.  The replay of
// a whole training step against the buffer layout (gpt2_audit_step) uses it
// to check, on the CPU, that every access stays inside its tensor.
#pragma once
#include <stddef.h>

struct AuditSink {
    virtual ~AuditSink() = default;
    // bytes [p, p + bytes) are read (write = false) or written / updated
    virtual void range(const char *kernel, const char *operand, const void *p, size_t bytes, bool write) = 0;
};

AuditSink *audit_sink();  // null unless a replay runs on this thread
void set_audit_sink(AuditSink *sink);

// `count` elements of T from p (nothing for a null pointer or count <= 0)
template <class T>
inline void audit(AuditSink *a, const char *kernel, const char *operand, const T *p, long long count, bool write) {
    if (p && count > 0) a->range(kernel, operand, (const void *)p, (size_t)count * sizeof(T), write);
}
