// The thread's launch-audit sink (see audit.h).
#include "audit.h"

namespace {
thread_local AuditSink *g_sink = nullptr;
}

AuditSink *audit_sink() { return g_sink; }
void set_audit_sink(AuditSink *sink) { g_sink = sink; }
