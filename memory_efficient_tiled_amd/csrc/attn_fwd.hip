// attn_fwd.hip -- host side of the attention forward: argument checks, the
// tile and split plan, workspace, launches, and the C entry points.  The
// kernels are in attn_fwd_kernel.h (one translation unit per head
// dimension: attn_fwd_d<D>.hip).

#include "attn_fwd_kernel.h"
#include "attn_plan.h"

#include <stdlib.h>

#include <algorithm>
#include <mutex>

namespace {

using namespace attn_fwd_detail;
using namespace attn_planner;

thread_local int g_last_hip_error = 0;

struct DeviceInfo {
  bool init = false;
  bool gfx950 = false;
  int cus = 0;
  void* scratch = nullptr;  // this device's address of `scratch` (attn_fwd_noalloc)
  hipMemPool_t pool = nullptr;  // stream-ordered workspace pool (workspace_pool)
};
std::mutex g_dev_mu;
DeviceInfo g_dev[64];

// Split-KV partials of attn_fwd_noalloc, for callers that cannot allocate
// device memory.  Every device the library runs on holds its own copy, from
// the library's load until the process ends.  In host code this name is not
// a device address: host code uses only the address hipGetSymbolAddress
// returns on each device (scratch_address below).
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

int device_info(DeviceInfo* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return ATTN_EHIP;
  }
  if (dev < 0 || dev >= 64) return ATTN_EUNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.init) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
      g_last_hip_error = (int)e;
      return ATTN_EHIP;
    }
    d.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.cus = prop.multiProcessorCount;
    d.init = true;
  }
  *out = d;
  return d.gfx950 ? ATTN_OK : ATTN_EUNSUPPORTED;
}

// The current device's address of `scratch`, looked up once per device
// (with that device current) and kept.  ATTN_EHIP if the lookup fails.
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return ATTN_EHIP;
  }
  if (dev < 0 || dev >= 64) return ATTN_EUNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.scratch) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      g_last_hip_error = (int)e;
      (void)hipGetLastError();
      return ATTN_EHIP;
    }
    d.scratch = ptr;
  }
  *out = d.scratch;
  return ATTN_OK;
}

hipError_t launch_fwd(int D, int Dv, const Params& p, int cfg, bool causal, bool split,
                      bool strided, bool masked, bool bf16, hipStream_t st) {
  if (Dv != D)  // the (192, 128) pair
    return launch_fwd_d<192, 128>(p, cfg, causal, split, strided, masked, bf16, st);
  switch (D) {
    case 64: return launch_fwd_d<64, 64>(p, cfg, causal, split, strided, masked, bf16, st);
    case 80: return launch_fwd_d<80, 80>(p, cfg, causal, split, strided, masked, bf16, st);
    case 96: return launch_fwd_d<96, 96>(p, cfg, causal, split, strided, masked, bf16, st);
    case 256: return launch_fwd_d<256, 256>(p, cfg, causal, split, strided, masked, bf16, st);
    default: return launch_fwd_d<128, 128>(p, cfg, causal, split, strided, masked, bf16, st);
  }
}

// The merge of split partials, for output rows of Dv elements.
hipError_t launch_combine(int Dv, const Params& p, bool strided, bool bf16, hipStream_t st) {
  switch (Dv) {
    case 64: return launch_combine_d<64>(p, strided, bf16, st);
    case 80: return launch_combine_d<80>(p, strided, bf16, st);
    case 96: return launch_combine_d<96>(p, strided, bf16, st);
    case 256: return launch_combine_d<256>(p, strided, bf16, st);
    default: return launch_combine_d<128>(p, strided, bf16, st);
  }
}

// `noalloc`: take the split workspace from this device's `scratch` array
// (ATTN_ESCRATCH, before any launch, when the plan needs more) instead of
// the workspace pool.
int run(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv,
        int Nq, int Nkv, int D, int Dv, const Layout& L, float scale, int causal, int dtype,
        int num_splits, hipStream_t stream, const MaskArgs& M = MaskArgs(),
        bool noalloc = false) {
  int rc = validate(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, Dv, scale, causal, dtype, L, M);
  const bool masked = M.type != ATTN_MASK_NONE;
  if (rc != ATTN_OK) return rc;
  if (num_splits < 0) return ATTN_EINVAL;
  DeviceInfo di;
  rc = device_info(&di);
  if (rc != ATTN_OK) return rc;

  // From here on the launch's heads, rows and strides are the packed ones
  // when the G query heads of a KV head are packed.
  const Packing pk = packing(Hq, Hkv, Nq, D, Dv, L, M);
  const int Nq0 = Nq;
  Hq = pk.Hq;
  Nq = pk.Nq;
  const Plan pl = make_plan(B, Hq, Nq, Nkv, D, Dv, causal, num_splits, di.cus, masked);
  const long long split_wgs = (pl.tiles - pl.first_split) * pl.splits;
  // grid sizes are ints: whole tiles and pieces share one launch
  if (pl.first_split + split_wgs > INT32_MAX) return ATTN_EINVAL;

  Params p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (uint16_t*)out;
  const Layout& PL = pk.L;
  p.qsb = PL.q.b, p.qsh = PL.q.h, p.qsn = (int)PL.q.n;
  p.ksb = PL.k.b, p.ksh = PL.k.h, p.ksn = (int)PL.k.n;
  p.vsb = PL.v.b, p.vsh = PL.v.h, p.vsn = (int)PL.v.n;
  p.osb = PL.o.b, p.osh = PL.o.h, p.osn = (int)PL.o.n;
  p.lse = lse;
  p.opart = nullptr;
  p.lsepart = nullptr;
  p.Hq = Hq;
  p.Nq = Nq;
  p.Nkv = Nkv;
  p.G = Hq / Hkv;  // 1 when packed
  p.Hkv = Hkv;
  p.n_qtiles = pl.n_qtiles;
  p.n_splits = pl.splits;
  p.split_len = pl.split_len;
  p.row0 = (int)pl.row0;
  p.prows = (int)(pl.rows - pl.row0);
  // A masked score is -inf and must give a probability of exactly 0, so the
  // factor applied to scores stays positive: for scale 0 every finite score
  // times FLT_MIN rounds to a base-2 exponent of 0, as it should.
  p.c = fmaxf(fabsf(scale) * kLog2e, FLT_MIN);
  p.qsign = scale < 0.f ? 0x80008000u : 0u;
  p.coff = causal == ATTN_CAUSAL_BOTTOM_RIGHT ? Nkv - Nq0 : 0;
  p.pos_nq = pk.on ? Nq0 : 0;
  p.mask = (const uint8_t*)pk.M.ptr;
  p.msb = pk.M.sb, p.msh = pk.M.sh, p.msq = pk.M.sq;
  p.mask_mode = pk.M.type;
  p.cm = p.c;
  if (M.type == ATTN_MASK_ADD) p.c = 1.f;  // the mask step forms base-2 scores

  void* ws = nullptr;
  if (noalloc) {
    void* sp = nullptr;
    rc = scratch_address(&sp);
    if (rc != ATTN_OK) return rc;
    if (split_wgs > 0) {
      if (pl.workspace_bytes() > (size_t)ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ESCRATCH;
      p.opart = (float*)sp;
      p.lsepart = p.opart + (size_t)pl.splits * p.prows * Dv;
    }
  } else if (split_wgs > 0) {
    hipError_t e = attn_host::workspace_alloc(&ws, pl.workspace_bytes(), stream);
    if (e != hipSuccess || !ws) {
      g_last_hip_error = (int)e;
      (void)hipGetLastError();
      return ATTN_ENOMEM;
    }
    p.opart = (float*)ws;
    p.lsepart = p.opart + (size_t)pl.splits * p.prows * Dv;
  }

  const bool cz = causal != 0;
  const Layout C = contiguous_layout(Hq, Hkv, Nq, Nkv, D, Dv);
  auto same = [](const Strides& a, const Strides& b) { return a.b == b.b && a.h == b.h && a.n == b.n; };
  const bool strided =
      !(same(PL.q, C.q) && same(PL.k, C.k) && same(PL.v, C.v) && same(PL.o, C.o));
  const bool bf16 = dtype == ATTN_BF16;
  auto launch = [&](bool split) {
    return launch_fwd(D, Dv, p, pl.cfg, cz, split, strided, masked, bf16, stream);
  };

  // Whole tiles and the pieces of the remaining tiles run in one launch,
  // whole tiles first: the pieces take the slots of the tiles that finish
  // first instead of waiting for the last one.  Then the merge.
  hipError_t e = hipSuccess;
  p.n_whole = 0;
  if (split_wgs > 0) {
    p.n_whole = (int)pl.first_split;
    p.total = (int)(pl.first_split + split_wgs);
    p.tile0 = (int)pl.first_split;
    e = launch(true);
    if (e == hipSuccess) e = launch_combine(Dv, p, strided, bf16, stream);
  } else if (pl.first_split > 0) {
    p.total = (int)pl.first_split;
    p.tile0 = 0;
    e = launch(false);
  }
  if (ws) {
    hipError_t ef = hipFreeAsync(ws, stream);
    if (e == hipSuccess) e = ef;
  }
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return ATTN_EHIP;
  }
  return ATTN_OK;
}

// The library's stream-ordered workspace pool on the current device, created
// on first use.  Its release threshold is the maximum, so memory it has
// handed out stays mapped between calls: with the default pool (threshold
// 0) every stream or device synchronisation returned the workspace to the
// driver, and the next call after it mapped it again (the first video-DiT
// step after a synchronisation took 3.3-3.4 ms instead of 2.9).
hipError_t workspace_pool(hipMemPool_t* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.pool) {
    hipMemPoolProps props = {};
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool = nullptr;
    e = hipMemPoolCreate(&pool, &props);
    if (e != hipSuccess) return e;
    uint64_t keep = UINT64_MAX;
    e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
    if (e != hipSuccess) {
      (void)hipMemPoolDestroy(pool);
      return e;
    }
    d.pool = pool;
  }
  *out = d.pool;
  return hipSuccess;
}

}  // namespace

namespace attn_host {
int check_device(int* cus) {
  DeviceInfo di;
  const int rc = device_info(&di);
  if (cus) *cus = di.cus;
  return rc;
}
void set_last_hip_error(int e) { g_last_hip_error = e; }
hipError_t workspace_alloc(void** p, size_t bytes, hipStream_t st) {
  const char* f = getenv("ATTN_FAIL_WORKSPACE");
  if (f && f[0] == '1' && f[1] == '\0') {
    *p = nullptr;
    return hipErrorOutOfMemory;
  }
  hipMemPool_t pool = nullptr;
  const hipError_t e = workspace_pool(&pool);
  if (e != hipSuccess) return e;
  return hipMallocFromPoolAsync(p, bytes, pool, st);
}
void narrow_plan(int B, int Hq, int Nq, int Nkv, int D, int causal, int num_splits, int cus,
                 NarrowPlan* out) {
  // the masked plan always takes the narrow tile of its head dimension
  const Plan pl = make_plan(B, Hq, Nq, Nkv, D, D, causal, num_splits, cus, true);
  out->n_qtiles = pl.n_qtiles;
  out->splits = pl.splits;
  out->split_len = pl.split_len;
  out->tiles = pl.tiles;
  out->first_split = pl.first_split;
  out->row0 = pl.row0;
  out->rows = pl.rows;
}
}  // namespace attn_host

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
             int Hkv, int Nq, int Nkv, int D, float scale, int causal, int dtype, void* stream) {
  return run(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, D,
             contiguous_layout(Hq, Hkv, Nq, Nkv, D, D), scale, causal, dtype, 0,
             (hipStream_t)stream);
}

int attn_fwd_split(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                   int Hq, int Hkv, int Nq, int Nkv, int D, float scale, int causal, int dtype,
                   int num_splits, void* stream) {
  return run(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, D,
             contiguous_layout(Hq, Hkv, Nq, Nkv, D, D), scale, causal, dtype, num_splits,
             (hipStream_t)stream);
}

int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                     int Hq, int Hkv, int Nq, int Nkv, int D, float scale, int causal, int dtype,
                     int num_splits, void* stream) {
  return run(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, D,
             contiguous_layout(Hq, Hkv, Nq, Nkv, D, D), scale, causal, dtype, num_splits,
             (hipStream_t)stream, MaskArgs(), true);
}

}  // extern "C"

namespace {
// Strides from the C arrays (batch, head, sequence); NULL = contiguous.
Layout strided_layout(int Hq, int Hkv, int Nq, int Nkv, int D, int Dv, const long long* qs,
                      const long long* ks, const long long* vs, const long long* os) {
  Layout L = contiguous_layout(Hq, Hkv, Nq, Nkv, D, Dv);
  auto take = [](Strides& s, const long long* a) {
    if (a) s = Strides{a[0], a[1], a[2]};
  };
  take(L.q, qs);
  take(L.k, ks);
  take(L.v, vs);
  take(L.o, os);
  return L;
}
}  // namespace

extern "C" {

int attn_fwd_strided(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                     int Hq, int Hkv, int Nq, int Nkv, int D, const long long* q_stride,
                     const long long* k_stride, const long long* v_stride,
                     const long long* o_stride, float scale, int causal, int dtype,
                     int num_splits, void* stream) {
  const Layout L = strided_layout(Hq, Hkv, Nq, Nkv, D, D, q_stride, k_stride, v_stride, o_stride);
  return run(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, D, L, scale, causal, dtype, num_splits,
             (hipStream_t)stream);
}

int attn_fwd_check(const void* q, const void* k, const void* v, const void* out, const float* lse,
                   int B, int Hq, int Hkv, int Nq, int Nkv, int D, float scale, int causal,
                   int dtype) {
  return validate(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, D, scale, causal, dtype,
                  contiguous_layout(Hq, Hkv, Nq, Nkv, D, D));
}

int attn_fwd_strided_check(const void* q, const void* k, const void* v, const void* out,
                           const float* lse, int B, int Hq, int Hkv, int Nq, int Nkv, int D,
                           const long long* q_stride, const long long* k_stride,
                           const long long* v_stride, const long long* o_stride, float scale,
                           int causal, int dtype) {
  return validate(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, D, scale, causal, dtype,
                  strided_layout(Hq, Hkv, Nq, Nkv, D, D, q_stride, k_stride, v_stride, o_stride));
}

static MaskArgs mask_args(const void* mask, int mask_type, const long long* mask_stride) {
  MaskArgs m;
  m.ptr = mask;
  m.type = mask_type;
  if (mask_type != ATTN_MASK_NONE) {
    if (!mask_stride) {
      m.type = -1;  // rejected by validation
    } else {
      m.sb = mask_stride[0];
      m.sh = mask_stride[1];
      m.sq = mask_stride[2];
    }
  }
  return m;
}

int attn_fwd_masked(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                    int Hq, int Hkv, int Nq, int Nkv, int D, const long long* q_stride,
                    const long long* k_stride, const long long* v_stride,
                    const long long* o_stride, const void* mask, int mask_type,
                    const long long* mask_stride, float scale, int causal, int dtype,
                    int num_splits, void* stream) {
  const Layout L = strided_layout(Hq, Hkv, Nq, Nkv, D, D, q_stride, k_stride, v_stride, o_stride);
  return run(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, D, L, scale, causal, dtype, num_splits,
             (hipStream_t)stream, mask_args(mask, mask_type, mask_stride));
}

int attn_fwd_masked_check(const void* q, const void* k, const void* v, const void* out,
                          const float* lse, int B, int Hq, int Hkv, int Nq, int Nkv, int D,
                          const long long* q_stride, const long long* k_stride,
                          const long long* v_stride, const long long* o_stride,
                          const void* mask, int mask_type, const long long* mask_stride,
                          float scale, int causal, int dtype) {
  return validate(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, D, scale, causal, dtype,
                  strided_layout(Hq, Hkv, Nq, Nkv, D, D, q_stride, k_stride, v_stride, o_stride),
                  mask_args(mask, mask_type, mask_stride));
}

int attn_fwd_dv(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
                int Hkv, int Nq, int Nkv, int D, int Dv, const long long* q_stride,
                const long long* k_stride, const long long* v_stride, const long long* o_stride,
                const void* mask, int mask_type, const long long* mask_stride, float scale,
                int causal, int dtype, int num_splits, void* stream) {
  const Layout L = strided_layout(Hq, Hkv, Nq, Nkv, D, Dv, q_stride, k_stride, v_stride, o_stride);
  return run(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, Dv, L, scale, causal, dtype, num_splits,
             (hipStream_t)stream, mask_args(mask, mask_type, mask_stride));
}

int attn_fwd_dv_check(const void* q, const void* k, const void* v, const void* out,
                      const float* lse, int B, int Hq, int Hkv, int Nq, int Nkv, int D, int Dv,
                      const long long* q_stride, const long long* k_stride,
                      const long long* v_stride, const long long* o_stride, const void* mask,
                      int mask_type, const long long* mask_stride, float scale, int causal,
                      int dtype) {
  return validate(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, Dv, scale, causal, dtype,
                  strided_layout(Hq, Hkv, Nq, Nkv, D, Dv, q_stride, k_stride, v_stride, o_stride),
                  mask_args(mask, mask_type, mask_stride));
}

// The planning queries take one head dimension: D = 192 stands for the
// (192, 128) pair, whose partial rows have 128 columns.
static int plan_dv(int D) { return D == 192 ? 128 : D; }

// Compute units of an MI355X, for the host-only workspace query.
constexpr int kMi355xCus = 256;

int attn_fwd_num_splits(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int causal, int dtype,
                        int num_cus) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nkv <= 0 || Hq % Hkv != 0) return ATTN_EINVAL;
  if (!head_dims_ok(D, plan_dv(D)) || (dtype != ATTN_F16 && dtype != ATTN_BF16))
    return ATTN_EINVAL;
  if (causal < 0 || causal > ATTN_CAUSAL_BOTTOM_RIGHT) return ATTN_EINVAL;
  return contiguous_plan(B, Hq, Hkv, Nq, Nkv, D, plan_dv(D), causal, 0, num_cus).splits;
}

int attn_fwd_plan(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int causal, int dtype,
                  int num_splits, int num_cus, attn_plan* plan) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nkv <= 0 || Hq % Hkv != 0) return ATTN_EINVAL;
  if (!head_dims_ok(D, plan_dv(D)) || (dtype != ATTN_F16 && dtype != ATTN_BF16))
    return ATTN_EINVAL;
  if (causal < 0 || causal > ATTN_CAUSAL_BOTTOM_RIGHT || num_splits < 0 || !plan)
    return ATTN_EINVAL;
  if ((long long)B * Hq * Nq > INT32_MAX || (long long)B * Hkv * Nkv > INT32_MAX)
    return ATTN_EINVAL;
  const Plan pl = contiguous_plan(B, Hq, Hkv, Nq, Nkv, D, plan_dv(D), causal, num_splits, num_cus);
  plan->tile_rows = kCfgs[pl.cfg].BM();
  plan->num_splits = pl.splits;
  plan->split_rows = pl.rows - pl.row0;
  plan->workspace_bytes = pl.workspace_bytes();
  return ATTN_OK;
}

// The plan depends on the number of KV heads only through GQA head
// packing; without it the query returns the largest workspace over every
// Hkv that divides Hq.
size_t attn_fwd_workspace_bytes(int B, int Hq, int Nq, int Nkv, int D, int causal) {
  if (B <= 0 || Hq <= 0 || Nq <= 0 || Nkv <= 0 || !head_dims_ok(D, plan_dv(D))) return 0;
  if (causal < 0 || causal > ATTN_CAUSAL_BOTTOM_RIGHT) return 0;
  if ((long long)B * Hq * Nq > INT32_MAX) return 0;
  size_t most = 0;
  for (int Hkv = 1; Hkv <= Hq; ++Hkv)
    if (Hq % Hkv == 0)
      most = std::max(most, contiguous_plan(B, Hq, Hkv, Nq, Nkv, D, plan_dv(D), causal, 0,
                                            kMi355xCus).workspace_bytes());
  return most;
}

const char* attn_strerror(int code) {
  switch (code) {
    case ATTN_OK: return "success";
    case ATTN_EINVAL: return "invalid argument";
    case ATTN_EUNSUPPORTED: return "unsupported device (gfx950 required)";
    case ATTN_ENOMEM: return "device workspace allocation failed";
    case ATTN_EHIP: return "HIP launch or runtime error";
    case ATTN_ESCRATCH:
      return "the split workspace exceeds the no-allocation scratch (ATTN_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown error code";
  }
}

int attn_last_hip_error(void) { return g_last_hip_error; }

int attn_workspace_pool(void** pool) {
  if (!pool) return ATTN_EINVAL;
  hipMemPool_t mp = nullptr;
  const hipError_t e = workspace_pool(&mp);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    (void)hipGetLastError();
    return ATTN_EHIP;
  }
  *pool = (void*)mp;
  return ATTN_OK;
}

}  // extern "C"
