// gdr_api.cpp -- the C ABI of libgdr: argument validation, launch planning,
// workspace sizes and the variable-length helpers.  Everything here is host
// code; validation finishes before the first HIP call, so every rejection can
// be exercised on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "gdr_internal.h"

namespace gdr {

static thread_local char g_last_error[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

// ---- per-kernel timing -----------------------------------------------------
volatile int g_profiling = 0;
namespace {
struct ProfRec {
  const char* name;
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
std::vector<ProfRec> g_prof;
}  // namespace

void profile_begin(hipStream_t st, const char* name) {
  ProfRec r;
  r.name = name;
  if (hipEventCreate(&r.start) != hipSuccess || hipEventCreate(&r.stop) != hipSuccess) return;
  (void)hipEventRecord(r.start, st);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof.push_back(r);
}

void profile_end(hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof.empty()) (void)hipEventRecord(g_prof.back().stop, st);
}

static gdr_status fail(gdr_status s, char* reason, size_t len, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  memcpy(g_last_error, buf, sizeof(buf));
  if (reason && len) {
    strncpy(reason, buf, len - 1);
    reason[len - 1] = '\0';
  }
  return s;
}

// Estimated scan time of a plan with P segments per sequence and VB 16-column
// state tiles per wave, in microseconds, calibrated on MI355X (256 CUs; one
// workgroup per CU in every pass but the forward transition pass at VB = 1,
// which fits two; a pass with more workgroups than slots runs in rounds).
// Per chunk step of one workgroup:
//   forward output pass 3.1 (VB = 1, wave-specialized; 2.55 in the
//   32-column form used when 64-column workgroups would fill at most 128
//   CUs) / 5.0 (VB = 2),
//   forward transition pass 2.7 / 3.0,
//   backward output pass (state and state-gradient scans in one launch):
//     state scan 2.4 / 5.5 and state-gradient scan 3.3 / 5.5; the launch
//     takes the longer of its total work spread over the CUs and one
//     state-gradient chain (no state scan when the forward's states are
//     given),
//   backward transition pass 4.5 / 4.2,
// one combine step 10 per scan, and 16 for the two extra launches of a split.
static double rounds(int64_t wgs, int64_t slots) {
  const int64_t r = (wgs + slots - 1) / slots;
  return r < 1 ? 1.0 : (double)r;
}

// fill: the mean chain over the longest (packed sequences whose scan blocks
// start the longest chains first, block_pos), else 1: the total work is
// spread over the CUs, never shorter than the longest chain.
static double bwd_out_cost(int64_t wgs_per_scan, int64_t chunks, int VB, bool states_given,
                           double fill) {
  // with the forward's states given only the state-gradient scan runs
  const double c1 = states_given ? 0.0 : (VB == 1 ? 2.4 : 5.5), c2 = VB == 1 ? 3.3 : 5.5;
  const double spread = (double)wgs_per_scan * (double)chunks * fill * (c1 + c2) / 256.0;
  const double chain = (double)chunks * c2;
  return spread > chain ? spread : chain;
}

// trans_given: the backward applies the forward's kept segment transitions,
// so its transition pass runs the value columns of every segment but the
// first, in a launch that fits two workgroups per CU at VB = 1.
static double plan_cost(int64_t units, int64_t maxch, int P, int VB, bool bwd, bool states_given,
                        bool trans_given, double fill) {
  const int64_t nvs0 = 2 / VB, nvs1 = 4 / VB;
  if (!bwd) {
    const bool narrow = VB == 1 && units * P * 2 <= 128;
    const double out = VB == 1 ? (narrow ? 2.55 : 3.1) : 5.0;
    if (P == 1 && fill < 1.0) {
      const double spread = (double)(units * nvs0) * (double)maxch * fill * out / 256.0;
      const double chain = (double)maxch * out;
      return spread > chain ? spread : chain;
    }
    if (P == 1) return (double)maxch * out * rounds(units * nvs0, 256);
    const int64_t sc = (maxch + P - 1) / P;
    // one end segment needs only its value columns, the inner ones everything
    const int64_t wg_aug = units * (nvs1 / 2 + (int64_t)(P - 2) * nvs1);
    const double aug = VB == 1 ? 2.7 : 3.0;
    return (double)sc * aug * rounds(wg_aug, VB == 1 ? 512 : 256) + 10.0 * (double)(P - 1) + 16.0 +
           (double)sc * out * rounds(units * P * nvs0, 256);
  }
  if (P == 1) return bwd_out_cost(units * nvs0, maxch, VB, states_given, fill);
  const int64_t sc = (maxch + P - 1) / P;
  const int64_t wg_aug = trans_given ? units * (int64_t)(P - 1) * (nvs1 / 2)
                                     : (states_given ? 1 : 2) * units *
                                           (nvs1 / 2 + (int64_t)(P - 2) * nvs1);
  const double aug = VB == 1 ? 4.5 : 4.2;
  const int64_t slots = (trans_given && VB == 1) ? 512 : 256;
  return (double)sc * aug * rounds(wg_aug, slots) +
         (states_given ? 10.0 : 20.0) * (double)(P - 1) + 16.0 +
         bwd_out_cost(units * P * nvs0, sc, VB, states_given, fill);
}

// Context-parallel plan along T: it depends only on shapes and flags (never
// on data), so every run of a problem, in either state layout, takes the same
// path.  One direction on its own, or, on the states path (a forward that
// keeps its packed chunk-start states, and the backward that takes them), one
// segment count for both directions, chosen for their sum: the backward then
// applies the forward's segment transitions instead of forming its own.
Plan make_plan(const gdr_problem* p, bool bwd, bool states_given) {
  const bool joint = bwd ? states_given : (p->h_packed != 0);
  Plan pl;
  pl.N = p->N;
  pl.total_chunks = 0;
  pl.max_len = 0;
  pl.nc_dense = 0;
  if (p->cu_seqlens_host) {
    for (int n = 0; n < p->N; ++n) {
      const int64_t L = (int64_t)p->cu_seqlens_host[n + 1] - p->cu_seqlens_host[n];
      pl.total_chunks += (L + kChunk - 1) / kChunk;
      if (L > pl.max_len) pl.max_len = L;
    }
  } else {
    pl.nc_dense = (p->T + kChunk - 1) / kChunk;
    pl.total_chunks = (int64_t)pl.nc_dense * p->B;
    pl.max_len = p->T;
  }
  const int64_t units = (int64_t)p->N * p->Hv;
  const int64_t maxch = (pl.max_len + kChunk - 1) / kChunk;
  // packed sequences with rank-ordered scan blocks (units a multiple of 8)
  const double fill = (p->cu_seqlens_host && units % 8 == 0 && maxch > 0)
                          ? (double)pl.total_chunks / ((double)p->N * (double)maxch)
                          : 1.0;
  pl.cp = 1;
  pl.vb = 2;
  double best = 1e300;
  const int fixed = p->cp_segments;
  // the forward's tile count on the states path: a forward that keeps packed
  // states writes them from the one-tile pass's output waves; the two-tile
  // pass would store them from its state chain (measured 681 -> 964 us for
  // one T=65536 sequence)
  const int vb_keep = p->wave_tiles > 0 ? p->wave_tiles : 1;
  for (int P = 1; P <= 16; P *= 2) {
    if (fixed > 0 && P != fixed) continue;
    if (fixed == 0 && P > 1 && maxch < 8 * P) continue;
    for (int VB = 1; VB <= 2; ++VB) {
      if (p->wave_tiles > 0 && VB != p->wave_tiles) continue;
      double c;
      if (!joint) {
        c = plan_cost(units, maxch, P, VB, bwd, states_given, false, fill);
      } else if (bwd) {  // VB is the backward's; the forward's is vb_keep
        c = plan_cost(units, maxch, P, vb_keep, false, false, false, fill) +
            plan_cost(units, maxch, P, VB, true, true, true, fill);
      } else {           // VB is the forward's; the backward takes its best
        if (VB != vb_keep) continue;
        double cb = 1e300;
        for (int VBb = 1; VBb <= 2; ++VBb) {
          if (p->wave_tiles > 0 && VBb != p->wave_tiles) continue;
          const double x = plan_cost(units, maxch, P, VBb, true, true, true, fill);
          if (x < cb) cb = x;
        }
        c = plan_cost(units, maxch, P, VB, false, false, false, fill) + cb;
      }
      // a split must win clearly: the model is coarse and splitting adds work
      c *= (P > 1 && fixed == 0) ? 1.1 : 1.0;
      if (c < best) {
        best = c;
        pl.cp = P;
        pl.vb = VB;
      }
    }
  }
  if (fixed > 0 && best == 1e300) {  // a segment count that is not a power of two
    pl.cp = fixed;
    pl.vb = p->wave_tiles > 0 ? p->wave_tiles : 1;
  }
  if (pl.cp > maxch) pl.cp = maxch > 0 ? (int)maxch : 1;
  return pl;
}

static bool is_half(gdr_dtype d) { return d == GDR_BF16 || d == GDR_FP16; }

static gdr_status validate(const gdr_problem* p, char* reason, size_t len) {
  if (!p) return fail(GDR_ERR_NULL, reason, len, "problem descriptor is NULL");
  if (p->K != kDim) return fail(GDR_ERR_HEAD_DIM, reason, len, "requires K=128, got %d", p->K);
  if (p->V != kDim) return fail(GDR_ERR_HEAD_DIM, reason, len, "requires V=128, got %d", p->V);
  if (!is_half(p->in_dtype))
    return fail(GDR_ERR_DTYPE, reason, len,
                "q/k/v must be bf16 or fp16 (got dtype code %d)", (int)p->in_dtype);
  if (p->g_dtype != p->in_dtype && p->g_dtype != GDR_FP32)
    return fail(GDR_ERR_DTYPE, reason, len, "g must have the input dtype or fp32 (got code %d)",
                (int)p->g_dtype);
  if (p->B < 1 || p->T < 1 || p->Hq < 1 || p->Hv < 1)
    return fail(GDR_ERR_SHAPE, reason, len, "sizes must be positive (B=%d T=%d Hq=%d Hv=%d)",
                p->B, p->T, p->Hq, p->Hv);
  if (p->Hq > p->Hv || p->Hv % p->Hq != 0)
    return fail(GDR_ERR_HEADS, reason, len,
                "value heads must be a multiple of q/k heads (Hq=%d Hv=%d)", p->Hq, p->Hv);
  if ((int64_t)p->B * p->T * p->Hv * kDim > ((int64_t)1 << 40))
    return fail(GDR_ERR_SHAPE, reason, len, "problem too large");
  if (!std::isfinite(p->scale)) return fail(GDR_ERR_ARG, reason, len, "scale must be finite");
  if (p->state_v_first != 0 && p->state_v_first != 1)
    return fail(GDR_ERR_ARG, reason, len, "state_v_first must be 0 or 1");
  if (p->cp_segments < 0) return fail(GDR_ERR_ARG, reason, len, "cp_segments must be >= 0");
  if (p->wave_tiles < 0 || p->wave_tiles > 2)
    return fail(GDR_ERR_ARG, reason, len, "wave_tiles must be 0, 1 or 2");
  if (p->use_qk_l2norm != 0 && p->use_qk_l2norm != 1)
    return fail(GDR_ERR_ARG, reason, len, "use_qk_l2norm must be 0 or 1");
  if (p->beta_sigmoid != 0 && p->beta_sigmoid != 1)
    return fail(GDR_ERR_ARG, reason, len, "beta_sigmoid must be 0 or 1");
  if (p->neg_eigval != 0 && p->neg_eigval != 1)
    return fail(GDR_ERR_ARG, reason, len, "neg_eigval must be 0 or 1");
  if (p->h_packed != 0 && p->h_packed != 1)
    return fail(GDR_ERR_ARG, reason, len, "h_packed must be 0 or 1");
  if (p->use_gate != 0 && p->use_gate != 1)
    return fail(GDR_ERR_ARG, reason, len, "use_gate must be 0 or 1");
  if (p->use_gate && !p->gate_A_log)
    return fail(GDR_ERR_NULL, reason, len, "use_gate needs gate_A_log");
  if (!p->use_gate && (p->gate_A_log || p->gate_dt_bias))
    return fail(GDR_ERR_ARG, reason, len, "gate parameters are given but use_gate is 0");
  const bool has_dev = p->cu_seqlens_dev != nullptr, has_host = p->cu_seqlens_host != nullptr;
  if (has_dev != has_host)
    return fail(GDR_ERR_VARLEN, reason, len,
                "cu_seqlens needs both the device and the host copy");
  if (has_dev) {
    if (p->B != 1)
      return fail(GDR_ERR_VARLEN, reason, len, "packed input needs B == 1, got %d", p->B);
    if (p->N < 1) return fail(GDR_ERR_VARLEN, reason, len, "N must be >= 1 with cu_seqlens");
    const int32_t* cu = p->cu_seqlens_host;
    if (cu[0] != 0) return fail(GDR_ERR_VARLEN, reason, len, "cu_seqlens[0] must be 0");
    for (int n = 0; n < p->N; ++n)
      if (cu[n + 1] < cu[n])
        return fail(GDR_ERR_VARLEN, reason, len, "cu_seqlens decreases at %d", n + 1);
    if (cu[p->N] != p->T)
      return fail(GDR_ERR_VARLEN, reason, len, "cu_seqlens[N]=%d must equal T=%d", cu[p->N],
                  p->T);
  } else if (p->N != p->B) {
    return fail(GDR_ERR_SHAPE, reason, len, "dense input needs N == B (N=%d B=%d)", p->N, p->B);
  }
  return GDR_OK;
}

static gdr_status check_device_cached() {
  static std::mutex mu;
  static int known[64];  // 0 unknown, 1 ok, 2 bad
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    set_error("no HIP device is available");
    return GDR_ERR_DEVICE;
  }
  std::lock_guard<std::mutex> lk(mu);
  if (dev < 64 && known[dev] == 1) return GDR_OK;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    set_error("hipGetDeviceProperties failed for device %d", dev);
    return GDR_ERR_DEVICE;
  }
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) known[dev] = ok ? 1 : 2;
  if (!ok) {
    set_error("device %d is %s; this library is built for gfx950 (MI355X)", dev,
              prop.gcnArchName);
    return GDR_ERR_DEVICE;
  }
  return GDR_OK;
}

template <typename I>
static gdr_status check_cu(const I* cu, int64_t n1) {
  if (!cu) {
    set_error("cu_seqlens is NULL");
    return GDR_ERR_NULL;
  }
  if (n1 < 1) {
    set_error("cu_seqlens needs at least one entry");
    return GDR_ERR_VARLEN;
  }
  if (cu[0] != 0) {
    set_error("cu_seqlens[0] must be 0");
    return GDR_ERR_VARLEN;
  }
  for (int64_t i = 1; i < n1; ++i)
    if (cu[i] < cu[i - 1]) {
      set_error("cu_seqlens decreases at %lld", (long long)i);
      return GDR_ERR_VARLEN;
    }
  return GDR_OK;
}

template <typename I>
static gdr_status lens_impl(const I* cu, int64_t n1, I* lens) {
  gdr_status s = check_cu(cu, n1);
  if (s != GDR_OK) return s;
  if (!lens && n1 > 1) {
    set_error("lens is NULL");
    return GDR_ERR_NULL;
  }
  for (int64_t i = 0; i + 1 < n1; ++i) lens[i] = cu[i + 1] - cu[i];
  return GDR_OK;
}

template <typename I>
static gdr_status indices_impl(const I* cu, int64_t n1, int64_t bt, I* out, int64_t* nc) {
  gdr_status s = check_cu(cu, n1);
  if (s != GDR_OK) return s;
  if (bt < 1) {
    set_error("chunk_size must be >= 1");
    return GDR_ERR_ARG;
  }
  if (!nc) {
    set_error("num_chunks is NULL");
    return GDR_ERR_NULL;
  }
  int64_t m = 0;
  for (int64_t i = 0; i + 1 < n1; ++i) {
    const int64_t c = ((int64_t)cu[i + 1] - cu[i] + bt - 1) / bt;
    for (int64_t j = 0; j < c; ++j, ++m)
      if (out) {
        out[2 * m] = (I)i;
        out[2 * m + 1] = (I)j;
      }
  }
  *nc = m;
  return GDR_OK;
}

template <typename I>
static gdr_status offsets_impl(const I* cu, int64_t n1, int64_t bt, I* offs, int64_t* total) {
  gdr_status s = check_cu(cu, n1);
  if (s != GDR_OK) return s;
  if (bt < 1) {
    set_error("chunk_size must be >= 1");
    return GDR_ERR_ARG;
  }
  if (!offs) {
    set_error("offsets is NULL");
    return GDR_ERR_NULL;
  }
  int64_t acc = 0;
  offs[0] = 0;
  for (int64_t i = 0; i + 1 < n1; ++i) {
    acc += ((int64_t)cu[i + 1] - cu[i] + bt - 1) / bt;
    offs[i + 1] = (I)acc;
  }
  if (total) *total = acc;
  return GDR_OK;
}

}  // namespace gdr

using namespace gdr;

extern "C" {

const char* gdr_status_string(gdr_status s) {
  switch (s) {
    case GDR_OK: return "GDR_OK";
    case GDR_ERR_NULL: return "GDR_ERR_NULL";
    case GDR_ERR_SHAPE: return "GDR_ERR_SHAPE";
    case GDR_ERR_HEAD_DIM: return "GDR_ERR_HEAD_DIM";
    case GDR_ERR_DTYPE: return "GDR_ERR_DTYPE";
    case GDR_ERR_HEADS: return "GDR_ERR_HEADS";
    case GDR_ERR_VARLEN: return "GDR_ERR_VARLEN";
    case GDR_ERR_WORKSPACE: return "GDR_ERR_WORKSPACE";
    case GDR_ERR_DEVICE: return "GDR_ERR_DEVICE";
    case GDR_ERR_HIP: return "GDR_ERR_HIP";
    case GDR_ERR_ARG: return "GDR_ERR_ARG";
  }
  return "GDR_UNKNOWN";
}

const char* gdr_last_error(void) { return g_last_error; }

gdr_status gdr_check_supported(const gdr_problem* p, char* reason, size_t reason_len) {
  gdr_status s = validate(p, reason, reason_len);
  if (s == GDR_OK && reason && reason_len) reason[0] = '\0';
  return s;
}

gdr_status gdr_check_device(void) { return check_device_cached(); }

// The unit q and k rows and their fp32 norms (q / k normalised in the
// kernel): 520 bytes per (token, q head), each part 256-byte aligned.
static size_t qk_rows_bytes(const gdr_problem* p) {
  const size_t rows = (size_t)p->B * p->T * p->Hq;
  return 2 * align256(rows * kDim * 2) + 2 * align256(rows * sizeof(float));
}

// gdr_chunk_fwd with q / k normalised and no user-layout h: the rows are
// normalised once (fwd_prep) into the workspace's tail, after the workspace
// of the problem without the option, which the rest then runs as
static size_t fwd_rows_offset(const gdr_problem* p) {
  gdr_problem pn = *p;
  pn.use_qk_l2norm = 0;
  return align256(fwd_workspace_bytes(&pn, make_plan(&pn, false)));
}

size_t gdr_chunk_fwd_workspace_size(const gdr_problem* p) {
  if (validate(p, nullptr, 0) != GDR_OK) return 0;
  size_t b = fwd_workspace_bytes(p, make_plan(p, false));
  if (p->use_qk_l2norm)  // the forms that run as a problem without the option
    b = std::max(b, fwd_rows_offset(p) + qk_rows_bytes(p));
  return b;
}

size_t gdr_chunk_bwd_workspace_size(const gdr_problem* p) {
  if (validate(p, nullptr, 0) != GDR_OK) return 0;
  return bwd_workspace_bytes(p, make_plan(p, true), false);
}

// The states path with q / k normalised in the kernel normalises the rows
// once, in the forward, and runs the rest as a problem without the option
// (the forward's scans and the backward's launches then take their
// loader-wave and data-scheduled forms); the rows and their norms are kept
// after the segment transitions in the caller's trans buffer.
static gdr_problem without_qk_norm(const gdr_problem* p) {
  gdr_problem pn = *p;
  pn.use_qk_l2norm = 0;
  return pn;
}

// Byte offsets in the trans buffer: the segment transitions, then (q / k
// normalised) the unit q and k rows and their fp32 1 / |x|.
struct TransLayout {
  size_t qn, kn, qinv, kinv, total;
};

static TransLayout trans_layout(const gdr_problem* p) {
  TransLayout t{0, 0, 0, 0, 0};
  if (!p->h_packed) return t;
  const gdr_problem pn = without_qk_norm(p);
  const Plan pl = make_plan(&pn, false);
  size_t o = pl.cp > 1 ? (size_t)pl.N * p->Hv * pl.cp * kDim * kDim * sizeof(float) : 0;
  if (p->use_qk_l2norm) {
    const size_t rows = (size_t)p->B * p->T * p->Hq;
    o = align256(o);
    t.qn = o;
    o += align256(rows * kDim * 2);
    t.kn = o;
    o += align256(rows * kDim * 2);
    t.qinv = o;
    o += align256(rows * sizeof(float));
    t.kinv = o;
    o += rows * sizeof(float);
  }
  t.total = o;
  return t;
}

size_t gdr_chunk_bwd_states_workspace_size(const gdr_problem* p) {
  if (validate(p, nullptr, 0) != GDR_OK) return 0;
  size_t b = bwd_workspace_bytes(p, make_plan(p, true, true), true);
  if (p->use_qk_l2norm) {  // with the forward's unit rows, or without them
    const gdr_problem pn = without_qk_norm(p);
    b = std::max(b, bwd_workspace_bytes(&pn, make_plan(&pn, true, true), true));
  }
  return b;
}

static gdr_status chunk_fwd(const gdr_problem* p, const void* q, const void* k, const void* v,
                            const void* g, const void* beta, const float* initial_state,
                            float* g_cum, void* A, void* o, void* h, float* trans,
                            float* final_state, void* workspace, size_t workspace_bytes,
                            void* stream, void* qn = nullptr, void* kn = nullptr,
                            float* qinv = nullptr, float* kinv = nullptr) {
  if (!q || !k || !v || !g || !beta || !g_cum || !A || !o)
    return fail(GDR_ERR_NULL, nullptr, 0, "a required forward pointer is NULL");
  const Plan pl = make_plan(p, false);
  const size_t need = fwd_workspace_bytes(p, pl);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(GDR_ERR_WORKSPACE, nullptr, 0, "forward workspace needs %zu bytes, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  const gdr_status s = check_device_cached();
  if (s != GDR_OK) return s;
  return launch_fwd(p, pl, q, k, v, g, beta, initial_state, g_cum, A, o, h,
                    pl.cp > 1 ? trans : nullptr, final_state, workspace, (hipStream_t)stream, qn,
                    kn, qinv, kinv);
}

gdr_status gdr_chunk_fwd(const gdr_problem* p, const void* q, const void* k, const void* v,
                         const void* g, const void* beta, const float* initial_state,
                         float* g_cum, void* A, void* o, void* h, float* final_state,
                         void* workspace, size_t workspace_bytes, void* stream) {
  const gdr_status s = validate(p, nullptr, 0);
  if (s != GDR_OK) return s;
  if (p->use_qk_l2norm && (!h || p->h_packed)) {
    // normalise the rows once (fwd_prep) into the workspace's tail and run
    // the rest without the option (the loader-wave output scan)
    const size_t off = fwd_rows_offset(p), need = off + qk_rows_bytes(p);
    if (!workspace || workspace_bytes < need)
      return fail(GDR_ERR_WORKSPACE, nullptr, 0, "forward workspace needs %zu bytes, got %zu",
                  need, workspace ? workspace_bytes : (size_t)0);
    const size_t rows = (size_t)p->B * p->T * p->Hq;
    char* t = reinterpret_cast<char*>(workspace) + off;
    char* kn = t + align256(rows * kDim * 2);
    char* qinv = kn + align256(rows * kDim * 2);
    char* kinv = qinv + align256(rows * sizeof(float));
    const gdr_problem pn = without_qk_norm(p);
    return chunk_fwd(&pn, q, k, v, g, beta, initial_state, g_cum, A, o, h, nullptr, final_state,
                     workspace, workspace_bytes, stream, t, kn, reinterpret_cast<float*>(qinv),
                     reinterpret_cast<float*>(kinv));
  }
  return chunk_fwd(p, q, k, v, g, beta, initial_state, g_cum, A, o, h, nullptr, final_state,
                   workspace, workspace_bytes, stream);
}

size_t gdr_chunk_trans_size(const gdr_problem* p) {
  if (validate(p, nullptr, 0) != GDR_OK || !p->h_packed) return 0;
  return trans_layout(p).total;
}

gdr_status gdr_chunk_fwd_states(const gdr_problem* p, const void* q, const void* k,
                                const void* v, const void* g, const void* beta,
                                const float* initial_state, float* g_cum, void* A, void* o,
                                void* h, float* trans, size_t trans_bytes, float* final_state,
                                void* workspace, size_t workspace_bytes, void* stream) {
  const gdr_status s = validate(p, nullptr, 0);
  if (s != GDR_OK) return s;
  if (!p->h_packed)
    return fail(GDR_ERR_ARG, nullptr, 0, "gdr_chunk_fwd_states keeps packed states: h_packed = 1");
  if (!h) return fail(GDR_ERR_NULL, nullptr, 0, "gdr_chunk_fwd_states needs h");
  const size_t tneed = gdr_chunk_trans_size(p);
  if (!trans && tneed > 0)
    return fail(GDR_ERR_NULL, nullptr, 0,
                "the plan splits sequences or q / k are normalised in the kernel: trans needs "
                "gdr_chunk_trans_size bytes");
  if (trans && trans_bytes < tneed)
    return fail(GDR_ERR_WORKSPACE, nullptr, 0, "trans needs %zu bytes, got %zu", tneed,
                trans_bytes);
  if (!p->use_qk_l2norm)
    return chunk_fwd(p, q, k, v, g, beta, initial_state, g_cum, A, o, h, trans, final_state,
                     workspace, workspace_bytes, stream);
  // fwd_prep normalises the rows once and keeps them; the rest runs without
  // the option
  const TransLayout t = trans_layout(p);
  char* tb = reinterpret_cast<char*>(trans);
  const gdr_problem pn = without_qk_norm(p);
  return chunk_fwd(&pn, q, k, v, g, beta, initial_state, g_cum, A, o, h, trans, final_state,
                   workspace, workspace_bytes, stream, tb + t.qn, tb + t.kn,
                   reinterpret_cast<float*>(tb + t.qinv), reinterpret_cast<float*>(tb + t.kinv));
}

static_assert(GDR_NOALLOC_SCRATCH_BYTES == kNoAllocScratchBytes, "header and library agree");

gdr_status gdr_chunk_fwd_noalloc(const gdr_problem* p, const void* q, const void* k,
                                 const void* v, const void* g, const void* beta,
                                 const float* initial_state, float* g_cum, void* A, void* o,
                                 void* h, float* final_state, void* stream) {
  gdr_status s = validate(p, nullptr, 0);
  if (s != GDR_OK) return s;
  if (!q || !k || !v || !g || !beta || !g_cum || !A || !o)
    return fail(GDR_ERR_NULL, nullptr, 0, "a required forward pointer is NULL");
  const Plan pl = make_plan(p, false);
  const size_t need = fwd_workspace_bytes(p, pl);
  if (need > kNoAllocScratchBytes)
    return fail(GDR_ERR_WORKSPACE, nullptr, 0,
                "the forward needs %zu bytes of workspace; the no-allocation forward holds at "
                "most %zu (call gdr_chunk_fwd with a workspace)",
                need, kNoAllocScratchBytes);
  s = check_device_cached();
  if (s != GDR_OK) return s;
  void* ws = nullptr;
  s = noalloc_scratch(&ws);
  if (s != GDR_OK) return s;
  return launch_fwd(p, pl, q, k, v, g, beta, initial_state, g_cum, A, o, h, nullptr, final_state,
                    ws, (hipStream_t)stream);
}

static gdr_status chunk_bwd(const gdr_problem* p, const void* q, const void* k, const void* v,
                            const float* g_cum, const void* graw, const void* beta, const void* A,
                            const void* do_, const float* dht, const float* initial_state,
                            const void* hstates, const float* trans, void* dq, void* dk,
                            void* dv, void* dbeta, void* dg, float* dh0, float* dA_log,
                            float* ddt_bias, void* workspace, size_t workspace_bytes,
                            void* stream, const float* qinv = nullptr,
                            const float* kinv = nullptr) {
  if (!q || !k || !v || !g_cum || !beta || !A || !do_ || !dq || !dk || !dv || !dbeta || !dg)
    return fail(GDR_ERR_NULL, nullptr, 0, "a required backward pointer is NULL");
  if (initial_state && !dh0)
    return fail(GDR_ERR_NULL, nullptr, 0, "dh0 is required when initial_state is given");
  const Plan pl = make_plan(p, true, hstates != nullptr);
  const size_t need = bwd_workspace_bytes(p, pl, hstates != nullptr);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(GDR_ERR_WORKSPACE, nullptr, 0, "backward workspace needs %zu bytes, got %zu",
                need, workspace ? workspace_bytes : (size_t)0);
  const gdr_status s = check_device_cached();
  if (s != GDR_OK) return s;
  return launch_bwd(p, pl, q, k, v, g_cum, graw, beta, A, do_, dht, initial_state, hstates,
                    pl.cp > 1 ? trans : nullptr, dq, dk, dv, dbeta, dg,
                    initial_state ? dh0 : nullptr, dA_log, ddt_bias, workspace,
                    (hipStream_t)stream, qinv, kinv);
}

gdr_status gdr_chunk_bwd(const gdr_problem* p, const void* q, const void* k, const void* v,
                         const float* g_cum, const void* beta, const void* A, const void* do_,
                         const float* dht, const float* initial_state, void* dq, void* dk,
                         void* dv, void* dbeta, void* dg, float* dh0, void* workspace,
                         size_t workspace_bytes, void* stream) {
  gdr_status s = validate(p, nullptr, 0);
  if (s != GDR_OK) return s;
  if (p->use_gate)
    return fail(GDR_ERR_ARG, nullptr, 0,
                "use_gate needs the gate input: call gdr_chunk_bwd_gate");
  return chunk_bwd(p, q, k, v, g_cum, nullptr, beta, A, do_, dht, initial_state, nullptr, nullptr,
                   dq, dk, dv, dbeta, dg, dh0, nullptr, nullptr, workspace, workspace_bytes,
                   stream);
}

gdr_status gdr_chunk_bwd_gate(const gdr_problem* p, const void* q, const void* k, const void* v,
                              const float* g_cum, const void* g, const void* beta, const void* A,
                              const void* do_, const float* dht, const float* initial_state,
                              void* dq, void* dk, void* dv, void* dbeta, void* dg, float* dh0,
                              float* dA_log, float* ddt_bias, void* workspace,
                              size_t workspace_bytes, void* stream) {
  gdr_status s = validate(p, nullptr, 0);
  if (s != GDR_OK) return s;
  if (!p->use_gate)
    return fail(GDR_ERR_ARG, nullptr, 0, "gdr_chunk_bwd_gate needs use_gate == 1");
  if (!g) return fail(GDR_ERR_NULL, nullptr, 0, "the gate input g is NULL");
  return chunk_bwd(p, q, k, v, g_cum, g, beta, A, do_, dht, initial_state, nullptr, nullptr, dq,
                   dk, dv, dbeta, dg, dh0, dA_log, ddt_bias, workspace, workspace_bytes, stream);
}

gdr_status gdr_chunk_bwd_states(const gdr_problem* p, const void* q, const void* k,
                                const void* v, const float* g_cum, const void* g,
                                const void* beta, const void* A, const void* do_,
                                const float* dht, const float* initial_state, const void* h,
                                const float* trans, size_t trans_bytes, void* dq, void* dk,
                                void* dv, void* dbeta, void* dg, float* dh0, float* dA_log,
                                float* ddt_bias, void* workspace, size_t workspace_bytes,
                                void* stream) {
  gdr_status s = validate(p, nullptr, 0);
  if (s != GDR_OK) return s;
  gdr_problem pk = *p;
  pk.h_packed = 1;
  if (trans) {
    // the transitions of the states path's plan, which the backward shares
    const size_t tneed = gdr_chunk_trans_size(&pk);
    if (trans_bytes < tneed)
      return fail(GDR_ERR_WORKSPACE, nullptr, 0, "trans needs %zu bytes, got %zu", tneed,
                  trans_bytes);
  }
  if (!h) return fail(GDR_ERR_NULL, nullptr, 0, "the forward's chunk-start states h are NULL");
  if (p->use_gate && !g) return fail(GDR_ERR_NULL, nullptr, 0, "the gate input g is NULL");
  if (!p->use_gate && (g || dA_log || ddt_bias))
    return fail(GDR_ERR_ARG, nullptr, 0, "g, dA_log and ddt_bias are for use_gate problems only");
  if (p->use_qk_l2norm && trans) {
    // the forward's unit rows: the backward runs without the option and maps
    // dq, dk back through the normalisation
    const TransLayout t = trans_layout(&pk);
    const char* tb = reinterpret_cast<const char*>(trans);
    const gdr_problem pn = without_qk_norm(p);
    return chunk_bwd(&pn, tb + t.qn, tb + t.kn, v, g_cum, p->use_gate ? g : nullptr, beta, A,
                     do_, dht, initial_state, h, trans, dq, dk, dv, dbeta, dg, dh0, dA_log,
                     ddt_bias, workspace, workspace_bytes, stream,
                     reinterpret_cast<const float*>(tb + t.qinv),
                     reinterpret_cast<const float*>(tb + t.kinv));
  }
  return chunk_bwd(p, q, k, v, g_cum, p->use_gate ? g : nullptr, beta, A, do_, dht,
                   initial_state, h, trans, dq, dk, dv, dbeta, dg, dh0, dA_log, ddt_bias,
                   workspace, workspace_bytes, stream);
}

gdr_status gdr_recurrent_fwd(const gdr_problem* p, const void* q, const void* k, const void* v,
                             const void* g, const void* beta, const float* initial_state,
                             void* o, float* final_state, void* stream) {
  gdr_status s = validate(p, nullptr, 0);
  if (s != GDR_OK) return s;
  if (!q || !k || !v || !g || !beta || !o)
    return fail(GDR_ERR_NULL, nullptr, 0, "a required recurrent-forward pointer is NULL");
  s = check_device_cached();
  if (s != GDR_OK) return s;
  return launch_recurrent(p, q, k, v, g, beta, initial_state, o, final_state, (hipStream_t)stream);
}

gdr_status gdr_plan_info(const gdr_problem* p, int backward, int32_t* cp_segments,
                         int32_t* wave_tiles) {
  gdr_status s = validate(p, nullptr, 0);
  if (s != GDR_OK) return s;
  // the backward of a forward that kept packed states takes them (no
  // recompute), which changes its plan
  const Plan pl = make_plan(p, backward != 0, backward != 0 && p->h_packed != 0);
  if (cp_segments) *cp_segments = pl.cp;
  if (wave_tiles) *wave_tiles = pl.vb;
  return GDR_OK;
}

gdr_status gdr_bwd_pipeline_info(const gdr_problem* p, int32_t* slices, int32_t* bounds,
                                 int32_t max_bounds) {
  gdr_status s = validate(p, nullptr, 0);
  if (s != GDR_OK) return s;
  int lo[9];
  const int S = bwd_pipe_bounds(p, make_plan(p, true, true), true, lo);
  if (slices) *slices = S;
  for (int i = 0; bounds && S > 0 && i <= S && i < max_bounds; ++i) bounds[i] = lo[i];
  return GDR_OK;
}

gdr_status gdr_profile_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_prof) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_prof.clear();
  g_profiling = enable ? 1 : 0;
  return GDR_OK;
}

int gdr_profile_read(char* names, size_t name_stride, double* total_ms, int* launches,
                     int max_entries) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  std::vector<std::string> keys;
  std::vector<double> tot;
  std::vector<int> cnt;
  for (auto& r : g_prof) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) == hipSuccess) (void)hipEventElapsedTime(&ms, r.start, r.stop);
    size_t i = 0;
    while (i < keys.size() && keys[i] != r.name) ++i;
    if (i == keys.size()) {
      keys.push_back(r.name);
      tot.push_back(0.0);
      cnt.push_back(0);
    }
    tot[i] += ms;
    cnt[i] += 1;
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_prof.clear();
  const int n = (int)keys.size() < max_entries ? (int)keys.size() : max_entries;
  for (int i = 0; i < n; ++i) {
    if (names && name_stride) {
      strncpy(names + i * name_stride, keys[i].c_str(), name_stride - 1);
      names[i * name_stride + name_stride - 1] = '\0';
    }
    if (total_ms) total_ms[i] = tot[i];
    if (launches) launches[i] = cnt[i];
  }
  return n;
}

gdr_status gdr_prepare_lens_i32(const int32_t* cu, int64_t n1, int32_t* lens) {
  return lens_impl(cu, n1, lens);
}
gdr_status gdr_prepare_lens_i64(const int64_t* cu, int64_t n1, int64_t* lens) {
  return lens_impl(cu, n1, lens);
}
gdr_status gdr_prepare_chunk_indices_i32(const int32_t* cu, int64_t n1, int64_t bt, int32_t* out,
                                         int64_t* nc) {
  return indices_impl(cu, n1, bt, out, nc);
}
gdr_status gdr_prepare_chunk_indices_i64(const int64_t* cu, int64_t n1, int64_t bt, int64_t* out,
                                         int64_t* nc) {
  return indices_impl(cu, n1, bt, out, nc);
}
gdr_status gdr_prepare_chunk_offsets_i32(const int32_t* cu, int64_t n1, int64_t bt,
                                         int32_t* offs, int64_t* total) {
  return offsets_impl(cu, n1, bt, offs, total);
}
gdr_status gdr_prepare_chunk_offsets_i64(const int64_t* cu, int64_t n1, int64_t bt,
                                         int64_t* offs, int64_t* total) {
  return offsets_impl(cu, n1, bt, offs, total);
}
gdr_status gdr_prepare_chunk_token_starts_i64(const int64_t* cu, int64_t n1, int64_t bt,
                                              int64_t* out, int64_t* nc) {
  gdr_status s = check_cu(cu, n1);
  if (s != GDR_OK) return s;
  if (bt < 1) {
    set_error("chunk_size must be >= 1");
    return GDR_ERR_ARG;
  }
  if (!nc) {
    set_error("num_chunks is NULL");
    return GDR_ERR_NULL;
  }
  int64_t m = 0;
  for (int64_t i = 0; i + 1 < n1; ++i) {
    for (int64_t t = cu[i]; t < cu[i + 1]; t += bt, ++m)
      if (out) {
        out[2 * m] = t;
        out[2 * m + 1] = m;
      }
  }
  *nc = m;
  return GDR_OK;
}

}  // extern "C"
