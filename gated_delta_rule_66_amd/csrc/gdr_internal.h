// gdr_internal.h -- host-side interface between the C ABI and the launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/gdr.h"

namespace gdr {

constexpr int kChunk = 64;
constexpr int kDim = 128;

// Launch plan derived from the problem on the host (no device access).
struct Plan {
  int N;              // sequences
  int64_t total_chunks;
  int nc_dense;       // chunks per sequence for dense batches (0 for packed)
  int64_t max_len;    // longest sequence
  int cp;             // context-parallel segments per sequence (1 = off)
  int vb;             // 16-column MFMA tiles per wave in the scans (1 or 2)
};

// states_given: the backward takes the forward's chunk states (no state
// scan).  A forward with p->h_packed and a backward with states_given plan
// jointly (one segment count for both, so that the backward can apply the
// forward's segment transitions).
Plan make_plan(const gdr_problem* p, bool bwd, bool states_given = false);

// Workspace layout helpers: every region is 256-byte aligned.
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t fwd_workspace_bytes(const gdr_problem* p, const Plan& pl);

// The no-allocation forward: its workspace is a file-scope device array of
// kNoAllocScratchBytes (gdr_fwd.hip); noalloc_scratch gives its address on the
// current device (resolved once per device with hipGetSymbolAddress).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
gdr_status noalloc_scratch(void** out);
size_t cp_workspace_bytes(const Plan& pl, int Hv);
// states_given: the forward's chunk-start states are an input (no state scan)
size_t bwd_workspace_bytes(const gdr_problem* p, const Plan& pl, bool states_given);
// The backward's pipeline: the number of slices S (0: one pass) and, in
// lo[0 .. S], the chunk each slice starts at (lo[S] = chunks per sequence);
// lo holds at least 9 entries.
int bwd_pipe_bounds(const gdr_problem* p, const Plan& pl, bool states_given, int* lo);

// trans: [N * Hv, cp, K, K] fp32, where the transition pass leaves every
// segment transition T_seg for the backward (NULL: kept in the workspace).
// qn, kn, qinv, kinv (all or none; p without use_qk_l2norm): fwd_prep
// normalises the q and k rows and keeps them there (the unit rows in q's
// layout, fp32 1 / |x| per (token, q head)); the scans read the unit rows.
gdr_status launch_fwd(const gdr_problem* p, const Plan& pl, const void* q, const void* k,
                      const void* v, const void* g, const void* beta, const float* h0,
                      float* gcum, void* A, void* o, void* h, float* trans, float* ht, void* ws,
                      hipStream_t st, void* qn = nullptr, void* kn = nullptr,
                      float* qinv = nullptr, float* kinv = nullptr);

// graw: the gate input (use_gate only, else NULL); dA_log, ddt_bias nullable.
// hstates: the forward's chunk-start states in the packed layout, or
// NULL to recompute them.  trans (with hstates, nullable): the forward's
// segment transitions for the same plan.
// qinv, kinv (nullable): q and k were normalised beforehand (qk_norm_rows)
// and p has use_qk_l2norm off; the gradient kernel maps dq, dk back through
// the normalisation with these per-(token, q head) 1 / |x|.
gdr_status launch_bwd(const gdr_problem* p, const Plan& pl, const void* q, const void* k,
                      const void* v, const float* gcum, const void* graw, const void* beta,
                      const void* A, const void* dO, const float* dht, const float* h0,
                      const void* hstates, const float* trans, void* dq, void* dk, void* dv,
                      void* dbeta, void* dg, float* dh0, float* dA_log, float* ddt_bias, void* ws,
                      hipStream_t st, const float* qinv = nullptr, const float* kinv = nullptr);

// Token-by-token recurrence (decode and other short inputs), no workspace.
gdr_status launch_recurrent(const gdr_problem* p, const void* q, const void* k, const void* v,
                            const void* g, const void* beta, const float* h0, void* o,
                            float* ht, hipStream_t st);

struct ScanArgs;
// The forward state scan (with the CP passes when pl.cp > 1).  mode 0 writes
// outputs, mode 2 only the chunk-start states.
template <typename T>
void launch_scan(const Plan& pl, ScanArgs a, int mode, hipStream_t st);

void set_error(const char* fmt, ...);

// Optional per-kernel timing (diagnostics): while enabled, every launch is
// bracketed by two HIP events recorded on its stream.
extern volatile int g_profiling;
void profile_begin(hipStream_t st, const char* name);
void profile_end(hipStream_t st);

#define GDR_LAUNCH(name, kernel, grid, block, st, ...)      \
  do {                                                      \
    if (::gdr::g_profiling) ::gdr::profile_begin(st, name); \
    hipLaunchKernelGGL(kernel, grid, block, 0, st, __VA_ARGS__); \
    if (::gdr::g_profiling) ::gdr::profile_end(st);         \
  } while (0)

}  // namespace gdr
