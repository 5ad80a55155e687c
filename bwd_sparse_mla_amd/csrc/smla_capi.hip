// C ABI of libsmla (see include/smla.h): argument checks, workspace layout
// and the launch sequence of each call.  No allocation, no synchronization.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "smla.h"
#include "smla_internal.h"

namespace smla {

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(int64_t s_q, int64_t s_kv, int heads, int topk, int kv_groups = 1) {
  if (kv_groups < 1 || kv_groups > 64) return fail(SMLA_ERR_SHAPE, "kv_groups must be in [1, 64]");
  if (s_q < 0 || s_kv < 1 || s_kv * kv_groups > MAX_SKV)
    return fail(SMLA_ERR_SHAPE, "s_q must be >= 0, s_kv >= 1 and s_kv * kv_groups < 2^24");
  if (heads < 1 || heads % kv_groups != 0)
    return fail(SMLA_ERR_SHAPE, "heads must be a positive multiple of kv_groups");
  const int hg = heads / kv_groups;
  if (hg != 8 && hg != 16 && hg != 32 && hg != 64 && hg != 128)
    return fail(SMLA_ERR_SHAPE, "heads per kv group must be 8, 16, 32, 64 or 128");
  if (topk < 1 || topk > MAX_TOPK) return fail(SMLA_ERR_SHAPE, "topk must be in [1, 16384]");
  if (s_q > (int64_t(1) << 31) / heads)
    return fail(SMLA_ERR_SHAPE, "s_q * heads must stay below 2^31");
  return SMLA_OK;
}

// The kernels' view of the rows.  With G kv groups, q [s_q, heads, 576] is
// [s_q G, heads / G, 576] (the pair (token, group) is one row of heads / G
// heads, reading index row s G + g of indices [s_q, G, topk]), and kv
// [s_kv, G, 576] is s_kv G flat rows (the planner maps a valid index j of
// group g to flat row j G + g for the gathers, and to block row g s_kv + j
// for the kv-major blocks of the dkv pass, so that a block holds one group's
// rows; finalize writes block row g s_kv + j to dkv row j G + g).  A query
// group is 64 rows; with 128 heads per kv
// group a row's heads are two groups, so the kernels run the 64-head form
// over twice the rows (the same memory: row (2r + j, h) is (r, 64 j + h)),
// half-row 2r + j reading index row r.
struct KernelShape {
  int64_t s_q;     // kernel rows of `heads` heads
  int64_t s_kv;    // flat kv rows
  int heads;
  int idx_shift;
};
KernelShape kernel_shape(int64_t s_q, int64_t s_kv, int heads, int kv_groups) {
  const int64_t r = s_q * kv_groups;
  const int hg = heads / kv_groups;
  if (hg == 128) return {2 * r, s_kv * kv_groups, 64, 1};
  return {r, s_kv * kv_groups, hg, 0};
}

// Group-major order: with G > 1 kv groups and fewer than 64 heads per group,
// a 64-row query group of token-major rows would hold rows of several kv
// groups (disjoint kv rows, each masked for the others).  The kernels then
// walk (group, token) pairs in group-major order (pair g S + s holds token
// s's heads of group g) and read and write q, out, dout, dq, the indices and
// the forward's lse at the caller's token-major rows (caller_token); only
// the backward's lse is permuted into the workspace (its staging area leads
// the workspace; the plan's layout follows it).
struct Stage {
  bool on = false;
  int hg = 0;
  size_t lse = 0, bytes = 0;
};
Stage make_stage(int64_t s_q, int heads, int kv_groups, int topk) {
  Stage st;
  st.hg = heads / kv_groups;
  if (kv_groups == 1 || st.hg >= 64 || s_q == 0) return st;
  st.on = true;
  const size_t rows = (size_t)s_q * heads;
  size_t o = 0;
  st.lse = o;  o = align256(o + rows * 4);
  st.bytes = o;
  return st;
}

// gfx950 check, cached per device ordinal.
int check_device() {
  static std::mutex mu;
  static int cache[64];  // 0 unknown, 1 ok, 2 unsupported
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(SMLA_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= 64) return fail(SMLA_ERR_DEVICE, "device ordinal out of range");
  {
    std::lock_guard<std::mutex> lk(mu);
    if (cache[dev] == 0) {
      hipDeviceProp_t prop;
      if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return fail(SMLA_ERR_HIP, "hipGetDeviceProperties failed");
      cache[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    }
    if (cache[dev] != 1) return fail(SMLA_ERR_DEVICE, "current device is not gfx950");
  }
  return SMLA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SMLA_OK;
  return fail(SMLA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Kernel timing for benchmarks: event pairs around each launch.
struct TimedLaunch {
  const char* name;
  hipEvent_t start, stop;
};
struct Timing {
  bool active = false;
  std::vector<hipEvent_t> pool;
  std::vector<TimedLaunch> recs;
  size_t next = 0;
};
Timing g_timing;

template <class F>
hipError_t timed(const char* name, hipStream_t s, F&& launch) {
  if (!g_timing.active || g_timing.next + 2 > g_timing.pool.size()) return launch();
  hipEvent_t a = g_timing.pool[g_timing.next], b = g_timing.pool[g_timing.next + 1];
  g_timing.next += 2;
  hipError_t e = hipEventRecord(a, s);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  e = hipEventRecord(b, s);
  if (e == hipSuccess) g_timing.recs.push_back({name, a, b});
  return e;
}

}  // namespace

// Scratch space of smla_fwd_noalloc: one buffer per device, resident from
// module load until the process ends.  In host code its name stands for a
// host-side symbol, not a device address: the device address is looked up
// (hipGetSymbolAddress, with the device current) on the first call on each
// device and kept in g_scratch_ptr, and only that pointer is handed to the
// kernels.
static __device__ __align__(256) char scratch[SMLA_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};   // device address of `scratch`, per device ordinal

// The current device's scratch buffer (its address looked up once per device).
int scratch_for_current_device(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(SMLA_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= 64) return fail(SMLA_ERR_DEVICE, "device ordinal out of range");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SMLA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return SMLA_OK;
}

}  // namespace

Plan make_plan(int64_t s_q, int64_t s_kv, int heads, int topk, bool backward, bool atomic,
               bool stored_p) {
  Plan p;
  p.s_q = s_q;
  p.s_kv = s_kv;
  p.heads = heads;
  p.topk = topk;
  p.T = tokens_per_group(heads);
  p.G = (s_q + p.T - 1) / p.T;
  p.NB = (s_kv + TILE_KV - 1) / TILE_KV;
  p.qcap = ((int64_t)p.T * topk + 63) / 64 * 64;  // a multiple of 64: aligned mask words
  const int64_t tk = (int64_t)p.T * topk;
  p.rcap = (int64_t)p.T * (tk < p.NB ? tk : p.NB);
  size_t o = 0;
  p.off_qcount = o;  o = align256(o + (size_t)p.G * 4);
  p.off_xcount = o;  o = align256(o + (size_t)p.G * 4);
  p.off_qrow = o;    o = align256(o + (size_t)p.G * p.qcap * 4);
  p.off_qmask = o;   o = align256(o + (size_t)p.G * p.qcap);
  p.off_gorder = o;  o = align256(o + (size_t)p.G * 4);
  p.off_xtotal = o;  o += 256;
  if (backward) {
    p.off_ktab = o;    o = align256(o + (size_t)p.NB * p.G * 8);
    p.off_krmask = o;  o = align256(o + (size_t)p.G * p.rcap * 8);
    p.off_delta = o;   o = align256(o + (size_t)s_q * heads * 4);
    p.off_clist = o;   o = align256(o + (size_t)p.NB * p.G * 8);
    p.off_nchunk = o;  o = align256(o + (size_t)p.NB * 4);
    p.off_ptouch = o;  o = align256(o + (size_t)(DKV_WGS + p.NB) * 2 * 8);
    p.off_spre = o;    o = align256(o + (size_t)(p.NB + 1) * 4);
    p.off_wstart = o;  o = align256(o + (size_t)DKV_WGS * 4);
    p.off_kbase = o;   o = align256(o + (size_t)p.NB * p.G * 4);
    p.off_korm = o;    o = align256(o + (size_t)p.NB * p.G * 8);
    p.off_cbase = o;   o = align256(o + (size_t)(p.NB + 1) * p.G * 4);
    p.off_cmask = o;   o = align256(o + (size_t)(p.NB + 1) * p.G * 8);
    // Mode-specific sizes go last, so the rest of the layout (and a plan
    // smla_plan built) is the same in every mode: the fp32 partials (64-row
    // units, or 128-row units in the stored-P form), the atomic mode's fp32
    // accumulator, then the stored-P form's P / dS buffer.
    {
      const int64_t ub = stored_p ? 2 : 1;
      const int64_t nu = (p.NB + ub - 1) / ub;
      p.off_part = o;
      o = align256(o + (size_t)(DKV_WGS + nu) * TILE_KV * ub * 576 * 4);
    }
    if (atomic) {
      p.off_acc32 = o;
      o = align256(o + (size_t)p.NB * TILE_KV * 576 * 4);
    }
    if (stored_p) {
      p.off_pds = o;
      o = align256(o + (size_t)p.G * p.qcap * 2 * GROUP_ROWS * 2);
    }
  }
  p.bytes = o;
  return p;
}

}  // namespace smla

using namespace smla;

extern "C" {

const char* smla_last_error(void) { return g_last_error.c_str(); }

int smla_version(void) { return SMLA_ABI_VERSION; }

int smla_device_supported(int device) {
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return 0;
  return std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
}

size_t smla_fwd_workspace_size_g(int64_t s_q, int64_t s_kv, int32_t heads, int32_t kv_groups,
                                 int32_t topk) {
  if (check_shape(s_q, s_kv, heads, topk, kv_groups) != SMLA_OK) return 0;
  const KernelShape k = kernel_shape(s_q, s_kv, heads, kv_groups);
  return make_plan(k.s_q, k.s_kv, k.heads, topk, false).bytes +
         make_stage(s_q, heads, kv_groups, topk).bytes;
}

size_t smla_fwd_workspace_size(int64_t s_q, int64_t s_kv, int32_t heads, int32_t topk) {
  return smla_fwd_workspace_size_g(s_q, s_kv, heads, 1, topk);
}

size_t smla_bwd_workspace_size_g(int64_t s_q, int64_t s_kv, int32_t heads, int32_t kv_groups,
                                 int32_t topk, uint32_t flags) {
  if (check_shape(s_q, s_kv, heads, topk, kv_groups) != SMLA_OK) return 0;
  const KernelShape k = kernel_shape(s_q, s_kv, heads, kv_groups);
  return make_plan(k.s_q, k.s_kv, k.heads, topk, true, (flags & SMLA_DKV_ATOMIC) != 0,
                   (flags & SMLA_DKV_STORED_P) != 0).bytes +
         make_stage(s_q, heads, kv_groups, topk).bytes;
}

size_t smla_bwd_workspace_size(int64_t s_q, int64_t s_kv, int32_t heads, int32_t topk,
                               uint32_t flags) {
  return smla_bwd_workspace_size_g(s_q, s_kv, heads, 1, topk, flags);
}

// Fills the planner's arguments for a workspace laid out by make_plan.
static PlanArgs plan_args(const Plan& p, const int32_t* indices, int64_t s_q, int64_t s_kv,
                          int topk, int idx_shift, int kv_groups, int64_t gmajor_s, char* ws,
                          bool backward) {
  PlanArgs pa{};
  pa.idx = indices;
  pa.idx_shift = idx_shift;
  pa.kv_groups = kv_groups;
  pa.gmajor_s = gmajor_s;
  pa.s_kv_idx = s_kv / kv_groups;
  pa.s_q = s_q;
  pa.s_kv = s_kv;
  pa.topk = topk;
  pa.G = p.G;
  pa.NB = p.NB;
  pa.qcap = p.qcap;
  pa.rcap = p.rcap;
  pa.qcount = reinterpret_cast<int*>(ws + p.off_qcount);
  pa.xcount = reinterpret_cast<int*>(ws + p.off_xcount);
  pa.xtotal = reinterpret_cast<int*>(ws + p.off_xtotal);
  pa.qrow = reinterpret_cast<int32_t*>(ws + p.off_qrow);
  pa.qmask = reinterpret_cast<uint8_t*>(ws + p.off_qmask);
  pa.ktab = backward ? reinterpret_cast<int2*>(ws + p.off_ktab) : nullptr;
  pa.krmask = backward ? reinterpret_cast<unsigned long long*>(ws + p.off_krmask) : nullptr;
  pa.kbase = backward ? reinterpret_cast<int*>(ws + p.off_kbase) : nullptr;
  pa.korm = backward ? reinterpret_cast<unsigned long long*>(ws + p.off_korm) : nullptr;
  return pa;
}

// Plan and order: the index plan of a workspace (backward layout when
// `backward`, which adds the kv-block records).  Nothing needs clearing
// first: the planner writes every entry of its structures, the order kernel
// the extra-entry total.
static int run_plan(const Plan& p, const PlanArgs& pa, int heads, bool backward, hipStream_t s) {
  int st;
  (void)backward;
  if (pa.s_q == 0) return hip_status(launch_fill_u32(pa.xtotal, 1, 0u, s), "fill");
  if ((st = hip_status(timed("plan", s, [&] { return launch_plan(pa, heads, s); }), "plan"))) return st;
  int* gorder = reinterpret_cast<int*>(reinterpret_cast<char*>(pa.qcount) - p.off_qcount + p.off_gorder);
  return hip_status(timed("order", s, [&] { return launch_order_groups(pa.qcount, pa.xcount, p.G, gorder, pa.xtotal, s); }), "order");
}

int smla_plan_g(const int32_t* indices, int64_t s_q, int64_t s_kv, int32_t heads,
                int32_t kv_groups, int32_t topk, void* workspace, size_t workspace_bytes,
                void* stream) {
  g_last_error.clear();
  int st = check_shape(s_q, s_kv, heads, topk, kv_groups);
  if (st) return st;
  if (s_q > 0 && !indices) return fail(SMLA_ERR_NULL, "indices is null");
  if (!aligned16(indices)) return fail(SMLA_ERR_ALIGN, "indices must be 16-byte aligned");
  const int64_t s_tok = s_q;
  const Stage sg = make_stage(s_q, heads, kv_groups, topk);
  const KernelShape k = kernel_shape(s_q, s_kv, heads, kv_groups);
  s_q = k.s_q;
  s_kv = k.s_kv;
  heads = k.heads;
  const Plan p = make_plan(s_q, s_kv, heads, topk, true);
  if (!workspace || workspace_bytes < p.bytes + sg.bytes)
    return fail(SMLA_ERR_WORKSPACE, "workspace smaller than smla_bwd_workspace_size()");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(SMLA_ERR_ALIGN, "workspace must be 256-byte aligned");
  if ((st = check_device())) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(workspace);
  char* ws = base + sg.bytes;
  return run_plan(p, plan_args(p, indices, s_q, s_kv, topk, k.idx_shift, kv_groups,
                               sg.on ? s_tok : 0, ws, true), heads, true, s);
}

int smla_plan(const int32_t* indices, int64_t s_q, int64_t s_kv, int32_t heads, int32_t topk,
              void* workspace, size_t workspace_bytes, void* stream) {
  return smla_plan_g(indices, s_q, s_kv, heads, 1, topk, workspace, workspace_bytes, stream);
}

}  // extern "C"

// The forward of smla_fwd_g (kv bf16 rows) and smla_fwd_fp8 (kv8 records).
static int fwd_impl(const void* q, const void* kv, const uint8_t* kv8, const int32_t* indices,
                    int64_t s_q, int64_t s_kv, int32_t heads, int32_t kv_groups, int32_t topk,
                    float sm_scale, void* out, float* lse, uint32_t flags, void* workspace,
                    size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!kv) kv = kv8;   // the checks below see the one kv given
  int st = check_shape(s_q, s_kv, heads, topk, kv_groups);
  if (st) return st;
  const uint32_t known = SMLA_PLAN_READY | (kv8 ? SMLA_FP8_POW2_SCALES : 0u);
  if (flags & ~known) return fail(SMLA_ERR_FLAGS, "unknown flag bits");
  if (!kv || (s_q > 0 && (!q || !indices || !out || !lse)))
    return fail(SMLA_ERR_NULL, "null tensor pointer");
  if (!aligned16(q) || !aligned16(kv) || !aligned16(indices) || !aligned16(out) || !aligned16(lse))
    return fail(SMLA_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  const int64_t s_tok = s_q;
  const Stage sg = make_stage(s_q, heads, kv_groups, topk);
  const KernelShape k = kernel_shape(s_q, s_kv, heads, kv_groups);
  s_q = k.s_q;
  s_kv = k.s_kv;
  heads = k.heads;
  // The forward fields of the workspace are a prefix of the backward layout,
  // so a plan built by smla_plan serves here too.
  const Plan p = make_plan(s_q, s_kv, heads, topk, false);
  if (!workspace || workspace_bytes < p.bytes + sg.bytes)
    return fail(SMLA_ERR_WORKSPACE, "workspace smaller than smla_fwd_workspace_size()");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(SMLA_ERR_ALIGN, "workspace must be 256-byte aligned");
  if ((st = check_device())) return st;
  if (s_q == 0) return SMLA_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(workspace);
  char* ws = base + sg.bytes;
  const PlanArgs pa = plan_args(p, indices, s_q, s_kv, topk, k.idx_shift, kv_groups,
                                sg.on ? s_tok : 0, ws, false);
  if (!(flags & SMLA_PLAN_READY) && (st = run_plan(p, pa, heads, false, s))) return st;

  FwdArgs fa{};
  fa.q = static_cast<const uint16_t*>(q);
  fa.kv = kv8 ? nullptr : static_cast<const uint16_t*>(kv);
  fa.kv8 = kv8;
  fa.s_q = s_q;
  fa.s_kv = s_kv;
  fa.scale_log2 = sm_scale * 1.4426950408889634f;
  fa.G = p.G;
  fa.qcap = p.qcap;
  fa.qcount = pa.qcount;
  fa.qrow = pa.qrow;
  fa.qmask = pa.qmask;
  fa.order = reinterpret_cast<int*>(ws + p.off_gorder);
  fa.out = static_cast<uint16_t*>(out);
  fa.lse = lse;
  fa.pair_s = s_tok;
  fa.pair_g = sg.on ? kv_groups : 1;
  if (kv8) {
    const int mode = (flags & SMLA_FP8_POW2_SCALES) ? 2 : 1;
    st = hip_status(timed("fwd_fp8", s, [&] { return launch_fwd(fa, heads, s, mode); }), "fwd_fp8");
  } else {
    st = hip_status(timed("fwd", s, [&] { return launch_fwd(fa, heads, s); }), "fwd");
  }
  return st;
}

extern "C" {

int smla_fwd_g(const void* q, const void* kv, const int32_t* indices, int64_t s_q, int64_t s_kv,
               int32_t heads, int32_t kv_groups, int32_t topk, float sm_scale, void* out,
               float* lse, uint32_t flags, void* workspace, size_t workspace_bytes, void* stream) {
  if (!kv) {
    g_last_error = "null tensor pointer";
    return SMLA_ERR_NULL;
  }
  return fwd_impl(q, kv, nullptr, indices, s_q, s_kv, heads, kv_groups, topk, sm_scale, out, lse,
                  flags, workspace, workspace_bytes, stream);
}

int smla_fwd_fp8(const void* q, const void* kv_fp8, const int32_t* indices, int64_t s_q,
                 int64_t s_kv, int32_t heads, int32_t kv_groups, int32_t topk, float sm_scale,
                 void* out, float* lse, uint32_t flags, void* workspace, size_t workspace_bytes,
                 void* stream) {
  if (!kv_fp8) {
    g_last_error = "null tensor pointer";
    return SMLA_ERR_NULL;
  }
  return fwd_impl(q, nullptr, static_cast<const uint8_t*>(kv_fp8), indices, s_q, s_kv, heads,
                  kv_groups, topk, sm_scale, out, lse, flags, workspace, workspace_bytes, stream);
}

int smla_fwd_ex(const void* q, const void* kv, const int32_t* indices, int64_t s_q, int64_t s_kv,
                int32_t heads, int32_t topk, float sm_scale, void* out, float* lse, uint32_t flags,
                void* workspace, size_t workspace_bytes, void* stream) {
  return smla_fwd_g(q, kv, indices, s_q, s_kv, heads, 1, topk, sm_scale, out, lse, flags,
                    workspace, workspace_bytes, stream);
}

int smla_fwd(const void* q, const void* kv, const int32_t* indices, int64_t s_q, int64_t s_kv,
             int32_t heads, int32_t topk, float sm_scale, void* out, float* lse,
             void* workspace, size_t workspace_bytes, void* stream) {
  return smla_fwd_g(q, kv, indices, s_q, s_kv, heads, 1, topk, sm_scale, out, lse, 0u, workspace,
                    workspace_bytes, stream);
}

int smla_fwd_noalloc(const void* q, const void* kv, const int32_t* indices, int64_t s_q,
                     int64_t s_kv, int32_t heads, int32_t topk, float sm_scale, void* out,
                     float* lse, void* stream) {
  g_last_error.clear();
  int st = check_shape(s_q, s_kv, heads, topk);
  if (st) return st;
  const size_t need = smla_fwd_workspace_size(s_q, s_kv, heads, topk);
  if (need > SMLA_NOALLOC_SCRATCH_BYTES)
    return fail(SMLA_ERR_WORKSPACE,
                "smla_fwd_noalloc: this shape needs " + std::to_string(need) +
                    " bytes of scratch, more than the library's " +
                    std::to_string(SMLA_NOALLOC_SCRATCH_BYTES) +
                    " bytes per device; call smla_fwd with a workspace");
  if (!kv) return fail(SMLA_ERR_NULL, "null tensor pointer");
  if ((st = check_device())) return st;
  void* ws = nullptr;
  if ((st = scratch_for_current_device(&ws))) return st;
  return fwd_impl(q, kv, nullptr, indices, s_q, s_kv, heads, 1, topk, sm_scale, out, lse, 0u, ws,
                  SMLA_NOALLOC_SCRATCH_BYTES, stream);
}

int smla_bwd_g(const void* q, const void* kv, const void* out, const void* dout,
               const int32_t* indices, const float* lse, int64_t s_q, int64_t s_kv, int32_t heads,
               int32_t kv_groups, int32_t topk, float sm_scale, void* dq, void* dkv,
               float* dkv_f32, uint32_t flags, void* workspace, size_t workspace_bytes,
               void* stream) {
  g_last_error.clear();
  int st = check_shape(s_q, s_kv, heads, topk, kv_groups);
  if (st) return st;
  if (!kv || (s_q > 0 && (!q || !out || !dout || !indices || !lse || !dq)))
    return fail(SMLA_ERR_NULL, "null tensor pointer");
  if (!dkv && !dkv_f32) return fail(SMLA_ERR_NULL, "dkv and dkv_f32 are both null");
  if (flags & ~(SMLA_DKV_ACCUMULATE | SMLA_DKV_ATOMIC | SMLA_PLAN_READY | SMLA_DKV_STORED_P))
    return fail(SMLA_ERR_FLAGS, "unknown flag bits");
  if ((flags & SMLA_DKV_ACCUMULATE) && !dkv_f32)
    return fail(SMLA_ERR_FLAGS, "SMLA_DKV_ACCUMULATE needs dkv_f32");
  const void* ptrs[] = {q, kv, out, dout, indices, lse, dq};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return fail(SMLA_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if ((dkv && !aligned16(dkv)) || (dkv_f32 && !aligned16(dkv_f32)))
    return fail(SMLA_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  const bool atomic = (flags & SMLA_DKV_ATOMIC) != 0;
  const bool stored_p = (flags & SMLA_DKV_STORED_P) != 0;
  const int64_t s_tok = s_q;
  const Stage sg = make_stage(s_q, heads, kv_groups, topk);
  const KernelShape k = kernel_shape(s_q, s_kv, heads, kv_groups);
  s_q = k.s_q;
  s_kv = k.s_kv;
  heads = k.heads;
  const Plan p = make_plan(s_q, s_kv, heads, topk, true, atomic, stored_p);
  if (!workspace || workspace_bytes < p.bytes + sg.bytes)
    return fail(SMLA_ERR_WORKSPACE, "workspace smaller than smla_bwd_workspace_size(flags)");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(SMLA_ERR_ALIGN, "workspace must be 256-byte aligned");
  if ((st = check_device())) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(workspace);
  char* ws = base + sg.bytes;
  if (sg.on) {   // a group-major copy of lse
    if ((st = hip_status(launch_permute_pairs(lse, base + sg.lse, s_tok, kv_groups, (int64_t)sg.hg * 4, true, s),
                         "permute")))
      return st;
    lse = reinterpret_cast<const float*>(base + sg.lse);
  }

  const PlanArgs pa = plan_args(p, indices, s_q, s_kv, topk, k.idx_shift, kv_groups,
                                sg.on ? s_tok : 0, ws, true);
  if (!(flags & SMLA_PLAN_READY) && (st = run_plan(p, pa, heads, true, s))) return st;
  int* gorder = reinterpret_cast<int*>(ws + p.off_gorder);

  BwdArgs ba{};
  ba.q = static_cast<const uint16_t*>(q);
  ba.kv = static_cast<const uint16_t*>(kv);
  ba.out = static_cast<const uint16_t*>(out);
  ba.dout = static_cast<const uint16_t*>(dout);
  ba.lse = lse;
  ba.s_q = s_q;
  ba.s_kv = s_kv;
  ba.scale = sm_scale;
  ba.scale_log2 = sm_scale * 1.4426950408889634f;
  ba.G = p.G;
  ba.NB = p.NB;
  ba.ub = stored_p ? 2 : 1;
  ba.NU = (p.NB + ba.ub - 1) / ba.ub;
  ba.qcap = p.qcap;
  ba.rcap = p.rcap;
  ba.qcount = pa.qcount;
  ba.xcount = pa.xcount;
  ba.xtotal = pa.xtotal;
  ba.qrow = pa.qrow;
  ba.qmask = pa.qmask;
  ba.ktab = pa.ktab;
  ba.krmask = pa.krmask;
  ba.gorder = gorder;
  ba.spre = reinterpret_cast<int*>(ws + p.off_spre);
  ba.wstart = reinterpret_cast<int*>(ws + p.off_wstart);
  ba.delta = reinterpret_cast<float*>(ws + p.off_delta);
  ba.clist = reinterpret_cast<int2*>(ws + p.off_clist);
  ba.nchunk = reinterpret_cast<int*>(ws + p.off_nchunk);
  ba.part = reinterpret_cast<float*>(ws + p.off_part);
  ba.ptouch = reinterpret_cast<unsigned long long*>(ws + p.off_ptouch);
  ba.acc32 = atomic ? reinterpret_cast<float*>(ws + p.off_acc32) : nullptr;
  ba.kbase = pa.kbase;
  ba.korm = pa.korm;
  ba.cbase = stored_p ? reinterpret_cast<int*>(ws + p.off_cbase) : nullptr;
  ba.cmask = stored_p ? reinterpret_cast<unsigned long long*>(ws + p.off_cmask) : nullptr;
  ba.pds = stored_p ? reinterpret_cast<uint16_t*>(ws + p.off_pds) : nullptr;
  ba.dq = static_cast<uint16_t*>(dq);
  ba.pair_s = s_tok;
  ba.pair_g = sg.on ? kv_groups : 1;
  ba.kvg = kv_groups;
  ba.kvs = s_kv / kv_groups;
  ba.dkv = static_cast<uint16_t*>(dkv);
  ba.dkv_f32 = dkv_f32;
  ba.accumulate = (flags & SMLA_DKV_ACCUMULATE) ? 1 : 0;
  if (s_q > 0 && (st = hip_status(timed("bwd_dq", s, [&] { return launch_bwd_dq(ba, heads, s); }), "bwd_dq"))) return st;
  if ((st = hip_status(timed("dkv_schedule", s, [&] { return launch_dkv_schedule(ba, s_q > 0, s); }), "dkv_schedule"))) return st;
  if (atomic && (st = hip_status(timed("dkv_clear", s, [&] {
                   return launch_fill_u32(ba.acc32, (size_t)p.NB * TILE_KV * 576, 0u, s);
                 }), "dkv_clear")))
    return st;
  if ((st = hip_status(timed("bwd_dkv", s, [&] { return launch_bwd_dkv(ba, heads, s); }), "bwd_dkv"))) return st;
  if ((st = hip_status(timed("dkv_finalize", s, [&] { return launch_dkv_finalize(ba, heads, s); }), "dkv_finalize")))
    return st;
  return SMLA_OK;
}

int smla_bwd(const void* q, const void* kv, const void* out, const void* dout,
             const int32_t* indices, const float* lse, int64_t s_q, int64_t s_kv, int32_t heads,
             int32_t topk, float sm_scale, void* dq, void* dkv, float* dkv_f32, uint32_t flags,
             void* workspace, size_t workspace_bytes, void* stream) {
  return smla_bwd_g(q, kv, out, dout, indices, lse, s_q, s_kv, heads, 1, topk, sm_scale, dq, dkv,
                    dkv_f32, flags, workspace, workspace_bytes, stream);
}

int smla_topk_indices(const float* logits, int64_t s_q, int64_t s_kv, int64_t ld,
                      const int32_t* ks, const int32_t* ke, int32_t topk, int32_t* indices,
                      void* stream) {
  g_last_error.clear();
  if (s_q < 0 || s_kv < 1 || ld < s_kv || topk < 1 || topk > MAX_TOPK)
    return fail(SMLA_ERR_SHAPE, "need s_q >= 0, s_kv >= 1, ld >= s_kv, 1 <= topk <= 16384");
  if (s_q > 0 && (!logits || !ks || !ke || !indices)) return fail(SMLA_ERR_NULL, "null pointer");
  const void* ptrs[] = {logits, ks, ke, indices};
  for (const void* ptr : ptrs)
    if ((reinterpret_cast<uintptr_t>(ptr) & 3u) != 0)
      return fail(SMLA_ERR_ALIGN, "pointers must be 4-byte aligned");
  int st = check_device();
  if (st) return st;
  TopkArgs ta{};
  ta.logits = logits;
  ta.s_q = s_q;
  ta.s_kv = s_kv;
  ta.ld = ld;
  ta.ks = ks;
  ta.ke = ke;
  ta.topk = topk;
  ta.out = indices;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return hip_status(timed("topk", s, [&] { return launch_topk(ta, s); }), "topk");
}

static int nonfinite_call(void* x, const void* ref, int32_t dtype, int64_t n, unsigned long long* count,
                          bool replace, void* stream) {
  g_last_error.clear();
  if (dtype != SMLA_DTYPE_BF16 && dtype != SMLA_DTYPE_F32)
    return fail(SMLA_ERR_SHAPE, "dtype must be SMLA_DTYPE_BF16 or SMLA_DTYPE_F32");
  if (n < 0) return fail(SMLA_ERR_SHAPE, "n must be >= 0");
  if (!count) return fail(SMLA_ERR_NULL, "count is null");
  if (n > 0 && !x) return fail(SMLA_ERR_NULL, "x is null");
  if ((reinterpret_cast<uintptr_t>(count) & 7u) != 0)
    return fail(SMLA_ERR_ALIGN, "count must be 8-byte aligned");
  if (!aligned16(x) || !aligned16(ref)) return fail(SMLA_ERR_ALIGN, "x and ref must be 16-byte aligned");
  const int es = dtype == SMLA_DTYPE_BF16 ? 2 : 4;
  if (replace && ref && ref != x) {
    const uintptr_t xb = reinterpret_cast<uintptr_t>(x), rb = reinterpret_cast<uintptr_t>(ref);
    const uintptr_t bytes = (uintptr_t)n * es;
    if (xb < rb + bytes && rb < xb + bytes) return fail(SMLA_ERR_SHAPE, "ref overlaps x");
  }
  int st = check_device();
  if (st) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return hip_status(timed(replace ? "nonfinite_replace" : "nonfinite_count", s,
                          [&] { return launch_nonfinite(x, ref, n, es, replace, count, s); }),
                    "nonfinite");
}

int smla_nonfinite_count(const void* x, int32_t dtype, int64_t n, unsigned long long* count,
                         void* stream) {
  return nonfinite_call(const_cast<void*>(x), nullptr, dtype, n, count, false, stream);
}

int smla_nonfinite_replace(void* x, const void* ref, int32_t dtype, int64_t n,
                           unsigned long long* count, void* stream) {
  return nonfinite_call(x, ref, dtype, n, count, true, stream);
}

int smla_validate_indices(const int32_t* indices, int64_t s_q, int32_t topk, int64_t s_kv,
                          unsigned long long* n_bad, void* stream) {
  g_last_error.clear();
  if (!n_bad) return fail(SMLA_ERR_NULL, "n_bad is null");
  if (s_q < 0 || topk < 1 || s_kv < 1) return fail(SMLA_ERR_SHAPE, "bad sizes");
  if (s_q > 0 && !indices) return fail(SMLA_ERR_NULL, "indices is null");
  if ((reinterpret_cast<uintptr_t>(n_bad) & 7u) != 0)
    return fail(SMLA_ERR_ALIGN, "n_bad must be 8-byte aligned");
  int st = check_device();
  if (st) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return hip_status(
      timed("validate", s, [&] { return launch_validate(indices, s_q * topk, s_kv, n_bad, s); }),
      "validate");
}

int smla_timing_start(int max_launches) {
  g_last_error.clear();
  if (max_launches < 1 || max_launches > (1 << 20))
    return fail(SMLA_ERR_SHAPE, "max_launches must be in [1, 2^20]");
  for (hipEvent_t e : g_timing.pool) (void)hipEventDestroy(e);
  g_timing.pool.clear();
  g_timing.recs.clear();
  g_timing.next = 0;
  for (int i = 0; i < 2 * max_launches; ++i) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return fail(SMLA_ERR_HIP, "hipEventCreate failed");
    g_timing.pool.push_back(e);
  }
  g_timing.active = true;
  return SMLA_OK;
}

int smla_timing_stop(void) {
  g_timing.active = false;
  return SMLA_OK;
}

int smla_timing_read(const char* kernel, int* launches, double* total_ms) {
  g_last_error.clear();
  if (!kernel || !launches || !total_ms) return fail(SMLA_ERR_NULL, "null argument");
  int n = 0;
  double tot = 0.0;
  for (const TimedLaunch& r : g_timing.recs) {
    if (std::strcmp(r.name, kernel) != 0) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess) return fail(SMLA_ERR_HIP, "event sync failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      return fail(SMLA_ERR_HIP, "hipEventElapsedTime failed");
    ++n;
    tot += ms;
  }
  *launches = n;
  *total_ms = tot;
  return SMLA_OK;
}

}  // extern "C"
