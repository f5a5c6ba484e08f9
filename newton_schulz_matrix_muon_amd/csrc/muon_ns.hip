// libmuon_ns.so: host side of the C ABI declared in include/muon_ns.h.
//
// Validation happens before any HIP call. The planner lays out the caller's workspace,
// splits the batch into chunks that fit, and enqueues, per chunk:
//   prep (norm partials + the one internal copy of X, in the n x m orientation) -> finalize (scale, flags)
//   -> the product sequence of the chosen variant (gemm.hpp) with fused epilogues.
// Everything is asynchronous on the caller's stream; nothing here synchronises.

#include "muon_ns.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include "common.hpp"
#include "elementwise.hpp"
#include "gemm.hpp"
#include "adamw.hpp"

using namespace mns;

// Scratch space of muon_step_noalloc. In host code this name is only the handle that
// hipGetSymbolAddress resolves to the current GPU's copy; kernels receive that address.
static __device__ __align__(256) char scratch[MNS_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local int g_last_hip = 0;

// ------------------------------------------------------------------ launch timing
enum Kind { K_PREP = 0, K_FINALIZE, K_SYRK, K_SYMPROD, K_RECT, K_CAST, K_SQUARE, K_ADAMW, NKINDS };
const char* const kKindNames[NKINDS] = {"prep_norm", "finalize_norm", "gemm_syrk", "gemm_symprod",
                                        "gemm_rect", "cast", "gemm_square", "adamw"};

struct Timing {
  std::mutex mu;
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev[NKINDS];
  std::vector<hipEvent_t> pool;
};
Timing& timing() {
  static Timing* t = new Timing();  // never destroyed: events may outlive static teardown
  return *t;
}

hipEvent_t take_event(Timing& t) {
  if (!t.pool.empty()) {
    hipEvent_t e = t.pool.back();
    t.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Launch `f` (which enqueues exactly one kernel on `s`), with events around it when
// timing is on. Returns MNS_OK or MNS_ERR_HIP.
template <class F>
int launch(int kind, hipStream_t s, F&& f) {
  Timing& t = timing();
  hipEvent_t e0 = nullptr, e1 = nullptr;
  bool rec = false;
  {
    std::lock_guard<std::mutex> lk(t.mu);
    if (t.on) {
      e0 = take_event(t);
      e1 = take_event(t);
      rec = e0 && e1;
    }
  }
  if (rec) (void)hipEventRecord(e0, s);
  f();
  hipError_t err = hipGetLastError();
  if (rec) {
    (void)hipEventRecord(e1, s);
    std::lock_guard<std::mutex> lk(t.mu);
    t.ev[kind].emplace_back(e0, e1);
  }
  if (err != hipSuccess) {
    g_last_hip = (int)err;
    return MNS_ERR_HIP;
  }
  return MNS_OK;
}

// ------------------------------------------------------------------ validation helpers
bool valid_dtype(int dt) { return dt == F32 || dt == BF16 || dt == F16; }

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

int check_tensor(const mns_tensor* t, bool need_ptr = true) {
  if (!t) return MNS_ERR_ARG;
  if (need_ptr && !t->ptr) return MNS_ERR_ARG;
  if (!valid_dtype(t->dtype)) return MNS_ERR_DTYPE;
  if (t->batch < 1 || t->rows < 1 || t->cols < 1) return MNS_ERR_SHAPE;
  if (t->ld < t->cols) return MNS_ERR_SHAPE;
  if (t->batch > 1 && t->stride < t->rows * t->ld) return MNS_ERR_SHAPE;
  // kernel index arithmetic: per-matrix element offsets and dims fit in int32
  if (t->rows > (1 << 24) || t->cols > (1 << 24) || t->rows * t->ld > INT32_MAX) return MNS_ERR_SHAPE;
  if (t->batch > (1 << 24)) return MNS_ERR_SHAPE;
  return MNS_OK;
}

bool same_shape(const mns_tensor* a, const mns_tensor* b) {
  return a->batch == b->batch && a->rows == b->rows && a->cols == b->cols;
}

// byte range [lo, hi) touched by a tensor
void extent(const mns_tensor* t, uintptr_t* lo, uintptr_t* hi) {
  const int64_t last = (t->batch - 1) * t->stride + (t->rows - 1) * t->ld + t->cols;
  *lo = reinterpret_cast<uintptr_t>(t->ptr);
  *hi = *lo + (uintptr_t)(last * dtype_size(t->dtype));
}

bool overlap(const mns_tensor* a, const mns_tensor* b) {
  uintptr_t a0, a1, b0, b1;
  extent(a, &a0, &a1);
  extent(b, &b0, &b1);
  return a0 < b1 && b0 < a1;
}

struct NsConf {
  int steps;
  float coeff[64][3];
  float eps;
  int io_dt, it_dt;
  uint32_t restart;
};

int check_params(const mns_ns_params* p, int io_dt, NsConf* c, const mns_tensor* G, int ngroups) {
  if (!p) return MNS_ERR_ARG;
  if (p->steps < 1 || p->steps > 64) return MNS_ERR_ARG;
  if (!(p->eps >= 0.f) || !std::isfinite(p->eps)) return MNS_ERR_ARG;
  if (!valid_dtype(p->iter_dtype)) return MNS_ERR_DTYPE;
  if (io_dt == F32 && p->iter_dtype != F32) return MNS_ERR_DTYPE;
  if (io_dt != F32 && p->iter_dtype == F32) return MNS_ERR_DTYPE;
  c->steps = p->steps;
  for (int k = 0; k < p->steps; ++k) {
    const float dflt[3] = {3.4445f, -4.7750f, 2.0315f};
    for (int j = 0; j < 3; ++j) {
      const float v = p->coeffs ? p->coeffs[3 * k + j] : dflt[j];
      if (!std::isfinite(v)) return MNS_ERR_ARG;
      c->coeff[k][j] = v;
    }
  }
  c->eps = p->eps;
  c->io_dt = io_dt;
  c->it_dt = p->iter_dtype;
  c->restart = p->restart_mask;
  // the products address each operand matrix with 32-bit byte offsets (offsets from 2^31 up
  // are their zero-fill sentinel): one n x m iterate must span at most 2^31 bytes
  const int64_t es = std::max(dtype_size(io_dt), dtype_size(p->iter_dtype));
  for (int i = 0; i < ngroups; ++i) {
    const int64_t n = std::min(G[i].rows, G[i].cols), m = std::max(G[i].rows, G[i].cols);
    if (n * round_up(m, 8) * es > (int64_t(1) << 31)) return MNS_ERR_SHAPE;
  }
  return MNS_OK;
}

// ------------------------------------------------------------------ workspace plan
struct Geo {
  int n, m;        // oriented: n <= m
  bool trans;      // caller matrix is m x n (rows > cols)
  int64_t ldn, ldm;
  int prep_tiles, prep_tiles_x;
};

Geo geometry(const mns_tensor* G) {
  Geo g;
  g.trans = G->rows > G->cols;
  g.n = (int)std::min(G->rows, G->cols);
  g.m = (int)std::max(G->rows, G->cols);
  g.ldn = round_up(g.n, 8);
  g.ldm = round_up(g.m, 8);
  g.prep_tiles_x = (int)((G->cols + PREP_T - 1) / PREP_T);
  g.prep_tiles = g.prep_tiles_x * (int)((G->rows + PREP_T - 1) / PREP_T);
  return g;
}

struct Buf {
  size_t off = 0;
  int64_t per = 0;  // elements per matrix
  int dt = 0;
};

struct Layout {
  size_t total = 0;
  Buf svec, partials, X0, X1, A, Bm, R, Z, W, Qa, Qb;
};

// Restart bits that take effect: steps k = 1 .. K-1 (bit k).
bool restart_at(const NsConf& c, int k) { return k >= 1 && k < c.steps && k < 32 && ((c.restart >> k) & 1u); }
bool restarts_used(const NsConf& c) {
  for (int k = 1; k < c.steps && k < 32; ++k)
    if (restart_at(c, k)) return true;
  return false;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

Layout plan(int variant, const Geo& g, const NsConf& c, int64_t chunk) {
  Layout L;
  size_t off = 0;
  auto add = [&](Buf& b, int64_t per, int dt_or_size, bool raw_bytes = false) {
    b.off = off;
    b.per = per;
    b.dt = raw_bytes ? -1 : dt_or_size;
    const size_t es = raw_bytes ? (size_t)dt_or_size : (size_t)dtype_size(dt_or_size);
    off = align256(off + (size_t)chunk * (size_t)per * es);
  };
  const int io = c.io_dt, it = c.it_dt;
  const int qdt = dtype_size(io) >= dtype_size(it) ? io : it;
  add(L.svec, 1, 4, true);
  add(L.partials, g.prep_tiles, 8, true);
  // X (n x ldm, row-major) is the only copy of an iterate: the rectangular products read it
  // k-major as their B operand, so no transposed copy is kept
  add(L.X0, (int64_t)g.n * g.ldm, io);
  const int64_t nn = (int64_t)g.n * g.ldn;
  if (variant == MNS_VARIANT_STANDARD) {
    add(L.X1, (int64_t)g.n * g.ldm, io);
    add(L.A, nn, it);
    add(L.Bm, nn, dtype_size(io) >= dtype_size(it) ? io : it);
  } else {
    if (restarts_used(c)) add(L.X1, (int64_t)g.n * g.ldm, io);
    add(L.R, nn, it);
    add(L.Z, nn, it);
    add(L.W, nn, it);
    add(L.Qa, nn, qdt);
    add(L.Qb, nn, qdt);
  }
  L.total = off;
  return L;
}

template <class T>
T* at(void* ws, const Buf& b) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(ws) + b.off);
}

int64_t pick_chunk(int variant, const Geo& g, const NsConf& c, int64_t batch, size_t ws_bytes) {
  const size_t one = plan(variant, g, c, 1).total;
  if (ws_bytes < one) return 0;
  const size_t per = plan(variant, g, c, 2).total - one;  // linear growth (+ alignment slack)
  int64_t b = per ? (int64_t)std::min<size_t>((size_t)batch, 1 + (ws_bytes - one) / per) : batch;
  b = std::max<int64_t>(1, std::min(b, batch));
  while (b > 1 && plan(variant, g, c, b).total > ws_bytes) --b;
  return b;
}

// ------------------------------------------------------------------ product launcher
struct Prod {
  const void* A = nullptr; int64_t lda = 0, sA = 0;
  const void* B = nullptr; int64_t ldb = 0, sB = 0;
  int M = 0, N = 0, K = 0, in_dt = 0;
  bool tri = false;
  bool bkm = false;  // B stored k-major: element (n, k) at B[k * ldb + n]
  const float* svec = nullptr; int spow = 0;
  float c0 = 0.f, c1 = 0.f, c2 = 1.f;
  const void* E = nullptr; int e_dt = 0; int64_t lde = 0, sE = 0; int e_rows = 0, e_cols = 0;
  void* C = nullptr; int c_dt = 0; int64_t ldc = 0, sC = 0; int c_rows = 0, c_cols = 0;
  void* Ct = nullptr; int ct_dt = 0; int64_t ldct = 0, sCt = 0; int ct_rows = 0, ct_cols = 0;
  void* W = nullptr; int w_dt = 0; int64_t ldw = 0, sW = 0; int w_trans = 0;
  void* U = nullptr; int u_dt = 0; int64_t ldu = 0, sU = 0;
  float u_scale = 0.f, lr = 0.f, wd_mul = 1.f;
  int32_t* flags = nullptr;
};

// Resident workgroups of a tile configuration on the current device (CUs x per-CU limit set
// by LDS and waves), cached per device.
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cached[dev] = cus;
  }
  return cached[dev];
}

template <class CFG>
int resident_slots() {
  const int by_lds = (160 * 1024) / CFG::LDS;
  const int by_waves = (4 * CFG::OCC) / (CFG::NT / 64);
  const int per_cu = std::max(1, std::min(by_lds, by_waves));
  return device_cus() * per_cu;
}

// Tile rows a full product's tile walk covers before moving one tile column right.
constexpr int kGroupM = 8;

template <typename T, class CFG, int EPI>
void launch_epi(int shape, dim3 grid, dim3 block, hipStream_t s, const GemmBatch& b) {
  if (shape == 3) hipLaunchKernelGGL((gemm_nt_kernel<T, 3, CFG, EPI>), grid, block, 0, s, b);
  else if (shape == 2) hipLaunchKernelGGL((gemm_nt_kernel<T, 2, CFG, EPI>), grid, block, 0, s, b);
  else if (shape == 1) hipLaunchKernelGGL((gemm_nt_kernel<T, 1, CFG, EPI>), grid, block, 0, s, b);
  else hipLaunchKernelGGL((gemm_nt_kernel<T, 0, CFG, EPI>), grid, block, 0, s, b);
}

template <typename T, class CFG>
void launch_half(int shape, int epi, dim3 grid, dim3 block, hipStream_t s, const GemmBatch& b) {
  switch (epi) {
    case 1: launch_epi<T, CFG, 1>(shape, grid, block, s, b); break;
    case 2: launch_epi<T, CFG, 2>(shape, grid, block, s, b); break;
    case 3: launch_epi<T, CFG, 3>(shape, grid, block, s, b); break;
    case 4: launch_epi<T, CFG, 4>(shape, grid, block, s, b); break;
    case 6: launch_epi<T, CFG, 6>(shape, grid, block, s, b); break;
    case 7: launch_epi<T, CFG, 7>(shape, grid, block, s, b); break;
    case 8: launch_epi<T, CFG, 8>(shape, grid, block, s, b); break;
    default: launch_epi<T, CFG, 0>(shape, grid, block, s, b); break;
  }
}

// Tile counts of one group's product for tile shape CFG.
template <class CFG>
int set_tiles(const Prod& q, GemmArgs& a, int64_t batch) {
  const int cover_n = std::max({q.N, q.C ? q.c_cols : 0, q.Ct ? q.ct_rows : 0});
  const int cover_m = std::max({q.M, q.C ? q.c_rows : 0, q.Ct ? q.ct_cols : 0});
  const int tm = (cover_m + CFG::BM - 1) / CFG::BM;
  const int tn = (cover_n + CFG::BN - 1) / CFG::BN;
  if (q.tri) {
    const int nt = std::max(tm, tn);
    a.tiles_m = a.tiles_n = nt;
    a.tiles_per_mat = nt * (nt + 1) / 2;
    a.group_m = 1;
  } else {
    a.tiles_m = tm;
    a.tiles_n = tn;
    a.tiles_per_mat = tm * tn;
    a.group_m = std::max(1, std::min(tm, kGroupM));
  }
  const int64_t nb = batch * (int64_t)a.tiles_per_mat;
  if (nb > INT32_MAX) return MNS_ERR_SHAPE;
  a.nblocks = (int)nb;
  return MNS_OK;
}

// One launch over ng groups that share the kernel instantiation (dtype, shape kind, epilogue).
template <class CFG>
int launch_prod(const Prod* qs, const GemmArgs* as, const int64_t* batches, int ng, int kind, hipStream_t s) {
  GemmBatch b;
  for (int i = 0; i < ng; ++i) {
    b.g[i] = as[i];
    if (int st = set_tiles<CFG>(qs[i], b.g[i], batches[i])) return st;
  }
  b.ng = ng;
  // tiles of the busiest XCD (each XCD takes part x of every group)
  int64_t xmax = 0;
  for (int x = 0; x < 8; ++x) {
    int64_t t = 0;
    for (int i = 0; i < ng; ++i) t += xcd_part_lo(b.g[i].nblocks, x + 1) - xcd_part_lo(b.g[i].nblocks, x);
    xmax = std::max(xmax, t);
  }
  if (8 * xmax > INT32_MAX) return MNS_ERR_SHAPE;
  // persistent grid (typed fast epilogue): 8 x (workgroups per XCD), at most the resident
  // workgroup slots; the generic epilogue runs one tile per workgroup, so its grid covers the
  // busiest XCD's share
  const int fast = as[0].fast_epi;
  const int64_t per_xcd = fast ? std::min<int64_t>(xmax, std::max(1, resident_slots<CFG>() / 8)) : xmax;
  dim3 grid((unsigned)(8 * std::max<int64_t>(1, per_xcd))), block(CFG::NT);
  const int shape = !qs[0].tri ? (qs[0].bkm ? 3 : 0) : (kind == K_SYRK ? 2 : 1);
  const int in_dt = qs[0].in_dt;
  return launch(kind, s, [&] {
    if (in_dt == F32) {
      if (fast) launch_epi<float, CFG, 5>(shape, grid, block, s, b);
      else launch_epi<float, CFG, 0>(shape, grid, block, s, b);
    } else if (in_dt == BF16) {
      launch_half<__bf16, CFG>(shape, fast, grid, block, s, b);
    } else {
      launch_half<_Float16, CFG>(shape, fast, grid, block, s, b);
    }
  });
}

// Tile choice: the 256 x 256 tile (1) when the product is large enough to fill the chip with
// it, else the 128 x 128 tile (0).
int tile_choice(const Prod& q, int64_t batch) {
  const int64_t t256 = batch * ((q.M + 255) / 256) * ((q.N + 255) / 256);
  if (q.in_dt == F32) return 0;
  if (q.M < 256 || t256 < 512) return 0;
  return 1;
}

GemmArgs gemm_args(const Prod& q, int64_t batch) {
  GemmArgs a;
  a.A = q.A; a.lda = q.lda; a.sA = q.sA;
  a.B = q.B; a.ldb = q.ldb; a.sB = q.sB;
  a.M = q.M; a.N = q.N; a.K = q.K;
  a.svec = q.svec; a.spow = q.spow;
  a.c0 = q.c0; a.c1 = q.c1; a.c2 = q.c2;
  a.E = q.E; a.e_dt = q.e_dt; a.lde = q.lde; a.sE = q.sE; a.e_rows = q.e_rows; a.e_cols = q.e_cols;
  a.C = q.C; a.c_dt = q.c_dt; a.ldc = q.ldc; a.sC = q.sC; a.c_rows = q.c_rows; a.c_cols = q.c_cols;
  a.Ct = q.Ct; a.ct_dt = q.ct_dt; a.ldct = q.ldct; a.sCt = q.sCt; a.ct_rows = q.ct_rows; a.ct_cols = q.ct_cols;
  a.W = q.W; a.w_dt = q.w_dt; a.ldw = q.ldw; a.sW = q.sW; a.w_trans = q.w_trans;
  a.U = q.U; a.u_dt = q.u_dt; a.ldu = q.ldu; a.sU = q.sU;
  a.u_scale = q.u_scale; a.lr = q.lr; a.wd_mul = q.wd_mul;
  a.flags = q.flags;
  a.tiles_m = a.tiles_n = a.tiles_per_mat = a.nblocks = a.group_m = 0;
  auto vec_ok = [&](const void* ptr, int64_t ld, int64_t stride) {
    return (int)(ptr && ld % 8 == 0 && (batch == 1 || stride % 8 == 0) &&
                 reinterpret_cast<uintptr_t>(ptr) % 16 == 0);
  };
  a.c_vec = vec_ok(q.C, q.ldc, q.sC);
  a.ct_vec = vec_ok(q.Ct, q.ldct, q.sCt);
  a.w_vec = vec_ok(q.W, q.ldw, q.sW);
  a.u_vec = vec_ok(q.U, q.ldu, q.sU);
  // typed fast epilogue: internal outputs only (C, optional C^T of the same dtype, no weight
  // update or flags), 8-aligned buffers and widths, E of a supported dtype pairing
  a.fast_epi = 0;
  const bool outs_ok = q.C && !q.W && !q.flags && a.c_vec && q.c_cols % 8 == 0 &&
                       (!q.Ct || (a.ct_vec && q.ct_dt == q.c_dt && q.ct_cols % 8 == 0));
  const int edt = q.E ? q.e_dt : q.c_dt;
  const bool e_ok = !q.E || (q.lde % 8 == 0 && q.sE % 8 == 0 && q.e_cols % 8 == 0 &&
                             reinterpret_cast<uintptr_t>(q.E) % 16 == 0);
  if (outs_ok && e_ok) {
    if (q.c_dt == F16 && edt == F16) a.fast_epi = 1;
    else if (q.c_dt == BF16 && edt == BF16) a.fast_epi = 2;
    else if (q.c_dt == F16 && edt == BF16) a.fast_epi = 3;
    else if (q.c_dt == BF16 && edt == F16) a.fast_epi = 4;
    else if (q.c_dt == F32 && edt == F32 && q.in_dt == F32) a.fast_epi = 5;
  }
  // the weight update alone (the last product of the Muon step): rectangular, no E, C, C^T,
  // U or diagonal term; W in 16-byte vectors along the direction the epilogue walks
  if (!q.tri && q.W && !q.U && !q.C && !q.Ct && !q.E && q.c0 == 0.f && q.in_dt != F32 && a.w_vec &&
      (q.w_trans ? q.M % 8 == 0 : q.N % 8 == 0)) {
    if (q.w_dt == BF16) a.fast_epi = 6;
    else if (q.w_dt == F16) a.fast_epi = 7;
    else if (q.w_dt == F32) a.fast_epi = 8;
  }
  return a;
}

// One product kind over ng groups (each a strided batch of its own shape): one launch when the
// groups agree on the kernel instantiation and tile shape, else one launch per group.
int run_prods(const Prod* qs, const int64_t* batches, int ng, int kind, hipStream_t s) {
  if (ng < 1 || ng > MNS_MAXG) return MNS_ERR_ARG;
  GemmArgs as[MNS_MAXG];
  int tc[MNS_MAXG];
  bool same = true;
  for (int i = 0; i < ng; ++i) {
    const Prod& q = qs[i];
    // the kernels address one operand matrix with 32-bit byte offsets and use offsets from
    // 2^31 up as the zero-fill sentinel: each operand matrix must span at most 2^31 bytes
    const int64_t es = dtype_size(q.in_dt);
    if ((int64_t)q.M * q.lda * es > (int64_t(1) << 31) ||
        (int64_t)(q.bkm ? q.K : q.N) * q.ldb * es > (int64_t(1) << 31))
      return MNS_ERR_SHAPE;
    as[i] = gemm_args(q, batches[i]);
    tc[i] = tile_choice(q, batches[i]);
    if (i && (q.in_dt != qs[0].in_dt || q.tri != qs[0].tri || q.bkm != qs[0].bkm ||
              as[i].fast_epi != as[0].fast_epi || tc[i] != tc[0]))
      same = false;
  }
  if (!same) {
    for (int i = 0; i < ng; ++i)
      if (int st = run_prods(qs + i, batches + i, 1, kind, s)) return st;
    return MNS_OK;
  }
  switch (tc[0]) {
    case 1: return launch_prod<Tile256>(qs, as, batches, ng, kind, s);
    default: return launch_prod<Tile128>(qs, as, batches, ng, kind, s);
  }
}

int run_prod(const Prod& q, int64_t batch, int kind, hipStream_t s) { return run_prods(&q, &batch, 1, kind, s); }

// Final destination of the last rectangular product.
struct FinalOut {
  const mns_tensor* O = nullptr;      // NS: the output batch
  const mns_tensor* W = nullptr;      // Muon step: weights (updated)
  const mns_tensor* U = nullptr;      // Muon step: optional update output
  float u_scale = 0.f, lr = 0.f, wd_mul = 1.f;
  int32_t* flags = nullptr;
};

void set_final(Prod& q, const FinalOut& f, const Geo& g, int64_t b0) {
  q.flags = f.flags ? f.flags + b0 : nullptr;
  if (f.O) {
    const int es = dtype_size(f.O->dtype);
    void* base = reinterpret_cast<char*>(f.O->ptr) + b0 * f.O->stride * es;
    if (!g.trans) {
      q.C = base; q.c_dt = f.O->dtype; q.ldc = f.O->ld; q.sC = f.O->stride;
      q.c_rows = g.n; q.c_cols = g.m;
    } else {
      q.Ct = base; q.ct_dt = f.O->dtype; q.ldct = f.O->ld; q.sCt = f.O->stride;
      q.ct_rows = g.m; q.ct_cols = g.n;
    }
  }
  if (f.W) {
    q.W = reinterpret_cast<char*>(f.W->ptr) + b0 * f.W->stride * dtype_size(f.W->dtype);
    q.w_dt = f.W->dtype; q.ldw = f.W->ld; q.sW = f.W->stride; q.w_trans = g.trans;
    q.u_scale = f.u_scale; q.lr = f.lr; q.wd_mul = f.wd_mul;
    if (f.U) {
      q.U = reinterpret_cast<char*>(f.U->ptr) + b0 * f.U->stride * dtype_size(f.U->dtype);
      q.u_dt = f.U->dtype; q.ldu = f.U->ld; q.sU = f.U->stride;
    }
  }
}

// Symmetric n x n product C = A . B^T (B symmetric) with the Newton-Schulz epilogue.
Prod sym_prod(const void* A, const void* B, int in_dt, const Geo& g, void* C, int c_dt) {
  Prod q;
  q.A = A; q.lda = g.ldn; q.sA = (int64_t)g.n * g.ldn;
  q.B = B; q.ldb = g.ldn; q.sB = (int64_t)g.n * g.ldn;
  q.M = g.n; q.N = g.n; q.K = g.n; q.in_dt = in_dt; q.tri = true;
  q.C = C; q.c_dt = c_dt; q.ldc = g.ldn; q.sC = (int64_t)g.n * g.ldn;
  q.c_rows = g.n; q.c_cols = (int)g.ldn;
  return q;
}

// Full n x n product C = A . B^T (no symmetry assumed: both triangles are computed).
Prod square_prod(const void* A, const void* B, int in_dt, const Geo& g, void* C, int c_dt) {
  Prod q = sym_prod(A, B, in_dt, g, C, c_dt);
  q.tri = false;
  return q;
}

// Gram product C = s^spow X X^T of the n x m row-major X.
Prod gram_prod(const void* X, int io_dt, const Geo& g, void* C, int c_dt, const float* svec, int spow) {
  Prod q;
  q.A = X; q.lda = g.ldm; q.sA = (int64_t)g.n * g.ldm;
  q.B = X; q.ldb = g.ldm; q.sB = (int64_t)g.n * g.ldm;
  q.M = g.n; q.N = g.n; q.K = g.m; q.in_dt = io_dt; q.tri = true;
  q.C = C; q.c_dt = c_dt; q.ldc = g.ldn; q.sC = (int64_t)g.n * g.ldn;
  q.c_rows = g.n; q.c_cols = (int)g.ldn;
  q.svec = svec; q.spow = spow;
  return q;
}

// Rectangular C = L . X for an n x n L and the n x m row-major X, read k-major in place.
Prod rect_prod(const void* L, const void* X, int io_dt, const Geo& g) {
  Prod q;
  q.A = L; q.lda = g.ldn; q.sA = (int64_t)g.n * g.ldn;
  q.B = X; q.ldb = g.ldm; q.sB = (int64_t)g.n * g.ldm; q.bkm = true;
  q.M = g.n; q.N = g.m; q.K = g.n; q.in_dt = io_dt; q.tri = false;
  return q;
}

void set_internal_x_out(Prod& q, void* X, int x_dt, const Geo& g) {
  q.C = X; q.c_dt = x_dt; q.ldc = g.ldm; q.sC = (int64_t)g.n * g.ldm;
  q.c_rows = g.n; q.c_cols = (int)g.ldm;
}

struct Source {
  const mns_tensor* G;
  const mns_tensor* M = nullptr;  // momentum (muon_step)
  float mu = 0.f;
  int nesterov = 0;
};

int run_prep(const Source& src, const Geo& g, const NsConf& c, const Layout& L, void* ws,
             int64_t b0, int64_t nb, int32_t* flags, hipStream_t s) {
  const mns_tensor* G = src.G;
  PrepArgs a;
  const int es = dtype_size(G->dtype);
  a.G = reinterpret_cast<const char*>(G->ptr) + b0 * G->stride * es;
  a.g_dt = G->dtype; a.ldg = G->ld; a.sg = G->stride;
  a.rows = (int)G->rows; a.cols = (int)G->cols;
  // X0 = G in the n x m orientation: a straight copy, or the transpose of an m x n G
  void* X0 = at<char>(ws, L.X0);
  a.out_same = nullptr; a.ld_same = 0; a.s_same = 0;
  a.out_tr = nullptr; a.ld_tr = 0; a.s_tr = 0;
  if (!g.trans) {
    a.out_same = X0; a.ld_same = g.ldm; a.s_same = (int64_t)g.n * g.ldm;
  } else {
    a.out_tr = X0; a.ld_tr = g.ldm; a.s_tr = (int64_t)g.n * g.ldm;
  }
  a.io_dt = c.io_dt;
  a.partials = at<double>(ws, L.partials);
  a.tiles_x = g.prep_tiles_x; a.tiles = g.prep_tiles;
  a.M = nullptr; a.ldm = 0; a.sm = 0; a.mu = 0.f; a.nesterov = 0;
  if (src.M) {
    a.M = reinterpret_cast<float*>(src.M->ptr) + b0 * src.M->stride;
    a.ldm = src.M->ld; a.sm = src.M->stride; a.mu = src.mu; a.nesterov = src.nesterov;
  }
  // vectorised path: every row and the momentum buffer 16-byte aligned, widths multiples of 8
  auto al = [](const void* ptr, int64_t ld, int64_t stride, int64_t batch) {
    return reinterpret_cast<uintptr_t>(ptr) % 16 == 0 && ld % 8 == 0 && (batch == 1 || stride % 8 == 0);
  };
  const bool vec = G->dtype == c.io_dt && G->cols % 8 == 0 && G->rows % 8 == 0 &&
                   al(G->ptr, G->ld, G->stride, G->batch) &&
                   (!src.M || al(src.M->ptr, src.M->ld, src.M->stride, src.M->batch));
  // without a transpose the aligned case streams whole rows; its partials (one per 4096
  // elements) never outnumber the 64 x 64 tiles the partial buffer is sized for
  const bool stream = vec && !g.trans;
  const int64_t sblocks = ((int64_t)G->rows * G->cols / 8 + PREP_SV - 1) / PREP_SV;
  const int tiles = stream ? (int)sblocks : g.prep_tiles;
  a.tiles = tiles;
  dim3 grid((unsigned)tiles, (unsigned)nb);
  int st = launch(K_PREP, s, [&] {
    if (!vec) hipLaunchKernelGGL(prep_kernel, grid, dim3(256), 0, s, a);
    else if (stream && c.io_dt == BF16) hipLaunchKernelGGL(prep_stream_kernel<__bf16>, grid, dim3(256), 0, s, a);
    else if (stream && c.io_dt == F16) hipLaunchKernelGGL(prep_stream_kernel<_Float16>, grid, dim3(256), 0, s, a);
    else if (stream) hipLaunchKernelGGL(prep_stream_kernel<float>, grid, dim3(256), 0, s, a);
    else if (c.io_dt == BF16) hipLaunchKernelGGL(prep_vec_kernel<__bf16>, grid, dim3(256), 0, s, a);
    else if (c.io_dt == F16) hipLaunchKernelGGL(prep_vec_kernel<_Float16>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(prep_vec_kernel<float>, grid, dim3(256), 0, s, a);
  });
  if (st) return st;
  double* part = at<double>(ws, L.partials);
  float* sv = at<float>(ws, L.svec);
  int32_t* fl = flags ? flags + b0 : nullptr;
  const float eps = c.eps;
  return launch(K_FINALIZE, s, [&] {
    hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)nb), dim3(256), 0, s, part, tiles, eps, sv, fl);
  });
}

// One group's share of a call: its geometry, workspace layout and base, the batch chunk
// [b0, b0 + nb) being processed, and where its results go.
struct Part {
  Geo g;
  Layout L;
  char* ws = nullptr;
  int64_t b0 = 0, nb = 0;
  Source src;
  FinalOut fo;
};

// Run one product kind over all parts: make(i) builds part i's product.
template <class F>
int run_all(const Part* P, int np, int kind, hipStream_t s, F&& make) {
  Prod qs[MNS_MAXG];
  int64_t nbs[MNS_MAXG];
  for (int i = 0; i < np; ++i) {
    qs[i] = make(i);
    nbs[i] = P[i].nb;
  }
  return run_prods(qs, nbs, np, kind, s);
}

int run_standard(const Part* P, int np, const NsConf& c, hipStream_t s) {
  const int io = c.io_dt, it = c.it_dt;
  struct Bufs { const float* sv; char* X[2]; char* A; char* Bm; } B[MNS_MAXG];
  for (int i = 0; i < np; ++i) {
    const Layout& L = P[i].L;
    void* ws = P[i].ws;
    B[i] = {at<float>(ws, L.svec), {at<char>(ws, L.X0), at<char>(ws, L.X1)}, at<char>(ws, L.A),
            at<char>(ws, L.Bm)};
  }
  int cur = 0;
  // X0 is the caller's values in the input dtype; every later X_k is normalised and is
  // stored in the iterate dtype (fp16 keeps 3 more mantissa bits than bf16 for B X).
  int xdt = io;
  for (int k = 1; k <= c.steps; ++k) {
    const float a_k = c.coeff[k - 1][0], b_k = c.coeff[k - 1][1], c_k = c.coeff[k - 1][2];
    const bool first = k == 1;
    // With fp16 or fp32 operands the a X term rides in the product, X <- (a I + b A + c A^2) X
    // (the guide's own form for the cubic, B = 1.5 I - 0.5 A), which spares the product's
    // epilogue a read of X. The first step multiplies the caller's X in its input dtype, and a
    // bf16 B would round the diagonal a + ... to 8 bits, so there a X stays an fp32 epilogue
    // term; likewise for bf16 iterates.
    const bool fold = !first && xdt != BF16;
    // A = X X^T (scaled by s^2 on the unnormalised first iterate)
    if (int st = run_all(P, np, K_SYRK, s, [&](int i) {
          return gram_prod(B[i].X[cur], xdt, P[i].g, B[i].A, it, B[i].sv, first ? 2 : 0);
        })) return st;
    // B = [a I +] b A + c A^2, stored in the dtype of X (the two are the operands of B X)
    if (int st = run_all(P, np, K_SYMPROD, s, [&](int i) {
          const Geo& g = P[i].g;
          Prod q = sym_prod(B[i].A, B[i].A, it, g, B[i].Bm, xdt);
          q.c0 = fold ? a_k : 0.f; q.c1 = b_k; q.c2 = c_k;
          q.E = B[i].A; q.e_dt = it; q.lde = g.ldn; q.sE = (int64_t)g.n * g.ldn; q.e_rows = g.n;
          q.e_cols = (int)g.ldn;
          return q;
        })) return st;
    // X <- s (a X + B X), or B X with the folded B
    if (int st = run_all(P, np, K_RECT, s, [&](int i) {
          const Geo& g = P[i].g;
          Prod q = rect_prod(B[i].Bm, B[i].X[cur], xdt, g);
          q.svec = B[i].sv; q.spow = first ? 1 : 0;
          if (!fold) {
            q.c1 = a_k; q.c2 = 1.f;
            q.E = B[i].X[cur]; q.e_dt = xdt; q.lde = g.ldm; q.sE = (int64_t)g.n * g.ldm; q.e_rows = g.n;
            q.e_cols = (int)g.ldm;
          }
          if (k < c.steps) set_internal_x_out(q, B[i].X[cur ^ 1], it, g);
          else set_final(q, P[i].fo, g, P[i].b0);
          return q;
        })) return st;
    cur ^= 1;
    xdt = it;
  }
  return MNS_OK;
}

// Copy the current Gram iterate of matrix 0 (n x ldn, iterate dtype) to trace (n x n fp32).
int trace_copy(const char* R, int it, const Geo& g, float* dst, hipStream_t s) {
  const int n = g.n;
  const int64_t ldn = g.ldn;
  const int64_t tot = (int64_t)n * n;
  const int blocks = (int)std::min<int64_t>(4096, (tot + 255) / 256);
  return launch(K_CAST, s, [&] {
    hipLaunchKernelGGL(copy2d_kernel, dim3(blocks), dim3(256), 0, s, (const void*)R, it, ldn,
                       (void*)dst, (int)F32, (int64_t)n, n, n);
  });
}

int run_gram(const Part* P, int np, const NsConf& c, hipStream_t s, float* trace = nullptr) {
  const int io = c.io_dt, it = c.it_dt;
  struct Bufs { const float* sv; char* X[2]; char* R; char* Z; char* Wb; char* Qbuf[2]; } B[MNS_MAXG];
  for (int i = 0; i < np; ++i) {
    const Layout& L = P[i].L;
    void* ws = P[i].ws;
    // X: n x ldm; a restart writes Q X into the other buffer (every output tile reads whole
    // columns of X, so the product cannot run in place)
    B[i] = {at<float>(ws, L.svec), {at<char>(ws, L.X0), L.X1.per ? at<char>(ws, L.X1) : nullptr},
            at<char>(ws, L.R), at<char>(ws, L.Z), at<char>(ws, L.W),
            {at<char>(ws, L.Qa), at<char>(ws, L.Qb)}};
  }
  int xc = 0;
  int xspow = 1;  // the current X is the unnormalised input: scale by s once
  int xdt = io;   // dtype of the current X; normalised restarts store it in the iterate dtype

  if (int st = run_all(P, np, K_SYRK, s, [&](int i) {
        return gram_prod(B[i].X[xc], xdt, P[i].g, B[i].R, it, B[i].sv, 2);
      })) return st;

  bool q_fresh = true;
  int qcur = 0;
  for (int k = 1; k <= c.steps; ++k) {
    const float a_k = c.coeff[k - 1][0], b_k = c.coeff[k - 1][1], c_k = c.coeff[k - 1][2];
    const bool restart = restart_at(c, k);
    const bool need_rect = restart || k == c.steps;
    // Z = a I + b R + c R^2 (straight into Q when Q is the identity)
    const bool zq = q_fresh;
    const int zdt = q_fresh && need_rect ? xdt : it;
    auto zdst = [&](int i) { return zq ? B[i].Qbuf[0] : B[i].Z; };
    if (int st = run_all(P, np, K_SYMPROD, s, [&](int i) {
          const Geo& g = P[i].g;
          Prod q = sym_prod(B[i].R, B[i].R, it, g, zdst(i), zdt);
          q.c0 = a_k; q.c1 = b_k; q.c2 = c_k;
          q.E = B[i].R; q.e_dt = it; q.lde = g.ldn; q.sE = (int64_t)g.n * g.ldn; q.e_rows = g.n;
          q.e_cols = (int)g.ldn;
          return q;
        })) return st;
    if (q_fresh) {
      qcur = 0;
      q_fresh = false;
    } else {
      // Q <- Z Q as a full product, in the order the steps act on X (Q_k = Z_k ... Z_1). In
      // rounded arithmetic the stored Z_j no longer commute exactly; keeping this ordered
      // product, instead of forcing Q symmetric, halves the error the half-precision
      // iterates add. Between updates the buffer holds Q^T, so both forms are NT products:
      // Q^T_new = Q^T Z, and Q_new = Z (Q^T)^T when Q goes on to multiply X.
      const int nxt = qcur ^ 1;
      if (int st = run_all(P, np, K_SQUARE, s, [&](int i) {
            return need_rect ? square_prod(zdst(i), B[i].Qbuf[qcur], it, P[i].g, B[i].Qbuf[nxt], xdt)
                             : square_prod(B[i].Qbuf[qcur], zdst(i), it, P[i].g, B[i].Qbuf[nxt], it);
          })) return st;
      qcur = nxt;
    }
    if (restart) {
      // X <- Q X (explicit), R <- X X^T, Q <- I
      if (int st = run_all(P, np, K_RECT, s, [&](int i) {
            Prod q = rect_prod(B[i].Qbuf[qcur], B[i].X[xc], xdt, P[i].g);
            q.svec = B[i].sv; q.spow = xspow;
            set_internal_x_out(q, B[i].X[xc ^ 1], it, P[i].g);
            return q;
          })) return st;
      xc ^= 1;
      xspow = 0;
      xdt = it;
      if (int st = run_all(P, np, K_SYRK, s, [&](int i) {
            return gram_prod(B[i].X[xc], xdt, P[i].g, B[i].R, it, B[i].sv, 0);
          })) return st;
      q_fresh = true;
    } else if (k < c.steps) {
      // W = R Z, R <- Z W
      if (int st = run_all(P, np, K_SYMPROD, s, [&](int i) {
            return sym_prod(B[i].R, zdst(i), it, P[i].g, B[i].Wb, it);
          })) return st;
      if (int st = run_all(P, np, K_SYMPROD, s, [&](int i) {
            return sym_prod(zdst(i), B[i].Wb, it, P[i].g, B[i].R, it);
          })) return st;
    }
    if (trace && k < c.steps) {
      const Geo& g = P[0].g;
      if (int st = trace_copy(B[0].R, it, g, trace + (int64_t)(k - 1) * g.n * g.n, s)) return st;
    }
  }
  // output = s^xspow Q X
  return run_all(P, np, K_RECT, s, [&](int i) {
    Prod q = rect_prod(B[i].Qbuf[qcur], B[i].X[xc], xdt, P[i].g);
    q.svec = B[i].sv; q.spow = xspow;
    set_final(q, P[i].fo, P[i].g, P[i].b0);
    return q;
  });
}

int run_parts(int variant, Part* P, int np, const NsConf& c, int32_t* const* flags, hipStream_t s,
              float* trace) {
  for (int i = 0; i < np; ++i) {
    if (int st = run_prep(P[i].src, P[i].g, c, P[i].L, P[i].ws, P[i].b0, P[i].nb, flags[i], s)) return st;
    P[i].fo.flags = flags[i];
  }
  return variant == MNS_VARIANT_STANDARD ? run_standard(P, np, c, s) : run_gram(P, np, c, s, trace);
}

// One group, processed in the largest batch chunks that fit the workspace.
int run_ns(int variant, const Source& src, const FinalOut& fo, const NsConf& c, void* ws,
           size_t ws_bytes, int32_t* flags, hipStream_t s, float* trace = nullptr) {
  Part P;
  P.g = geometry(src.G);
  const int64_t batch = src.G->batch;
  const int64_t chunk = pick_chunk(variant, P.g, c, batch, ws_bytes);
  if (chunk < 1) return MNS_ERR_WORKSPACE;
  P.L = plan(variant, P.g, c, chunk);
  P.ws = reinterpret_cast<char*>(ws);
  P.src = src;
  for (int64_t b0 = 0; b0 < batch; b0 += chunk) {
    P.b0 = b0;
    P.nb = std::min(chunk, batch - b0);
    P.fo = fo;
    int32_t* fl[1] = {flags};
    if (int st = run_parts(variant, &P, 1, c, fl, s, trace)) return st;
  }
  return MNS_OK;
}

// Workspace for processing ng groups side by side, each as one whole-batch chunk.
size_t grouped_bytes(int variant, int ng, const mns_tensor* G, const NsConf& c) {
  size_t tot = 0;
  for (int i = 0; i < ng; ++i) tot = align256(tot + plan(variant, geometry(&G[i]), c, G[i].batch).total);
  return tot;
}

// ng groups: side by side (every product one launch over all groups) when the workspace
// holds them all at once, else one group after another (each chunked as needed).
int run_groups(int variant, int ng, const Source* srcs, const FinalOut* fos, const NsConf& c,
               void* ws, size_t ws_bytes, int32_t* flags, hipStream_t s) {
  const mns_tensor* Gs[MNS_MAXG];
  int64_t foff[MNS_MAXG];
  int64_t off = 0;
  for (int i = 0; i < ng; ++i) {
    Gs[i] = srcs[i].G;
    foff[i] = off;
    off += srcs[i].G->batch;
  }
  size_t need = 0;
  for (int i = 0; i < ng; ++i) need = align256(need + plan(variant, geometry(Gs[i]), c, Gs[i]->batch).total);
  if (need > ws_bytes) {
    for (int i = 0; i < ng; ++i)
      if (int st = run_ns(variant, srcs[i], fos[i], c, ws, ws_bytes, flags ? flags + foff[i] : nullptr, s))
        return st;
    return MNS_OK;
  }
  Part P[MNS_MAXG];
  int32_t* fl[MNS_MAXG];
  size_t woff = 0;
  for (int i = 0; i < ng; ++i) {
    P[i].g = geometry(Gs[i]);
    P[i].L = plan(variant, P[i].g, c, Gs[i]->batch);
    P[i].ws = reinterpret_cast<char*>(ws) + woff;
    woff = align256(woff + P[i].L.total);
    P[i].b0 = 0;
    P[i].nb = Gs[i]->batch;
    P[i].src = srcs[i];
    P[i].fo = fos[i];
    fl[i] = flags ? flags + foff[i] : nullptr;
  }
  return run_parts(variant, P, ng, c, fl, s, nullptr);
}

int ns_entry(int variant, const mns_tensor* G, const mns_tensor* O, const mns_ns_params* p,
             void* ws, size_t ws_bytes, int32_t* flags, void* stream) {
  if (int st = check_tensor(G)) return st;
  if (int st = check_tensor(O)) return st;
  if (!same_shape(G, O)) return MNS_ERR_SHAPE;
  if (O->dtype != G->dtype) return MNS_ERR_DTYPE;
  if (overlap(G, O)) return MNS_ERR_ARG;
  NsConf c;
  if (int st = check_params(p, G->dtype, &c, G, 1)) return st;
  if (!ws) return MNS_ERR_WORKSPACE;
  Source src;
  src.G = G;
  FinalOut fo;
  fo.O = O;
  return run_ns(variant, src, fo, c, ws, ws_bytes, flags, reinterpret_cast<hipStream_t>(stream));
}

// Validation shared by the single and grouped Muon step.
int check_step(const mns_tensor* W, const mns_tensor* G, const mns_tensor* M, const mns_tensor* U_out) {
  if (int st = check_tensor(W)) return st;
  if (int st = check_tensor(G)) return st;
  if (int st = check_tensor(M)) return st;
  if (!same_shape(W, G) || !same_shape(M, G)) return MNS_ERR_SHAPE;
  if (M->dtype != F32) return MNS_ERR_DTYPE;
  if (U_out) {
    if (int st = check_tensor(U_out)) return st;
    if (!same_shape(U_out, G)) return MNS_ERR_SHAPE;
    if (overlap(U_out, W) || overlap(U_out, G) || overlap(U_out, M)) return MNS_ERR_ARG;
  }
  if (overlap(W, G) || overlap(W, M) || overlap(G, M)) return MNS_ERR_ARG;
  return MNS_OK;
}

int check_step_params(const mns_step_params* sp) {
  if (!sp) return MNS_ERR_ARG;
  if (sp->variant != MNS_VARIANT_STANDARD && sp->variant != MNS_VARIANT_GRAM) return MNS_ERR_ARG;
  const float vals[4] = {sp->lr, sp->momentum, sp->weight_decay, sp->scale_coeff};
  for (float v : vals)
    if (!std::isfinite(v)) return MNS_ERR_ARG;
  return MNS_OK;
}

void step_io(const mns_tensor* W, const mns_tensor* G, const mns_tensor* M, const mns_tensor* U_out,
             const mns_step_params* sp, Source* src, FinalOut* fo) {
  src->G = G;
  src->M = M;
  src->mu = sp->momentum;
  src->nesterov = sp->nesterov ? 1 : 0;
  fo->W = W;
  fo->U = U_out;
  fo->u_scale = sp->scale_coeff * (float)std::sqrt((double)std::max(W->rows, W->cols));
  fo->lr = sp->lr;
  fo->wd_mul = (float)(1.0 - (double)sp->lr * (double)sp->weight_decay);
}

// Any two of the listed buffers overlap.
bool any_overlap(const mns_tensor* const* t, int n) {
  for (int i = 0; i < n; ++i)
    for (int j = i + 1; j < n; ++j)
      if (t[i] && t[j] && overlap(t[i], t[j])) return true;
  return false;
}

// Device address of the GPU's copy of `scratch` for work on `stream`, looked up once per GPU
// with that GPU current.
int scratch_address(hipStream_t stream, void** out) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0, cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e == hipSuccess) e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_hip = (int)e;
    return MNS_ERR_HIP;
  }
  if (dev < 0 || dev >= 64) return MNS_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) {
      g_last_hip = (int)e;
      return MNS_ERR_HIP;
    }
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess || !a || back != hipSuccess) {
      g_last_hip = (int)(e != hipSuccess ? e : back);
      return MNS_ERR_HIP;
    }
    addr[dev] = a;
  }
  *out = addr[dev];
  return MNS_OK;
}

int run_adamw(int nt, void* const* params, const void* const* grads, float* const* m, float* const* v,
              const int64_t* numels, int dt, const mns_adamw_params* ap, hipStream_t s) {
  AdamTable t;
  t.lr = ap->lr;
  t.beta1 = ap->beta1;
  t.beta2 = ap->beta2;
  t.eps = ap->eps;
  t.wd_mul = (float)(1.0 - (double)ap->lr * (double)ap->weight_decay);
  t.bc1 = ap->bias_correction ? (float)(1.0 / (1.0 - std::pow((double)ap->beta1, ap->step))) : 1.f;
  t.bc2 = ap->bias_correction ? (float)(1.0 / (1.0 - std::pow((double)ap->beta2, ap->step))) : 1.f;
  int i = 0;
  while (i < nt) {
    int k = 0;
    int64_t blocks = 0;
    for (; i < nt && k < ADAM_MAXT; ++i) {
      if (numels[i] == 0) continue;
      const int64_t b = (numels[i] + ADAM_CHUNK - 1) / ADAM_CHUNK;
      if (blocks + b > INT32_MAX) break;
      t.p[k] = params[i];
      t.g[k] = grads[i];
      t.m[k] = m[i];
      t.v[k] = v[i];
      t.numel[k] = numels[i];
      t.blk_start[k] = (int)blocks;
      blocks += b;
      ++k;
    }
    if (k == 0) {
      if (i < nt && numels[i] > 0) return MNS_ERR_SHAPE;   // one tensor beyond INT32_MAX blocks
      continue;
    }
    t.blk_start[k] = (int)blocks;
    t.nt = k;
    if (int st = launch(K_ADAMW, s, [&] {
          if (dt == F32) hipLaunchKernelGGL(adamw_kernel<float>, dim3((unsigned)blocks), dim3(ADAM_BLOCK), 0, s, t);
          else if (dt == BF16) hipLaunchKernelGGL(adamw_kernel<__bf16>, dim3((unsigned)blocks), dim3(ADAM_BLOCK), 0, s, t);
          else hipLaunchKernelGGL(adamw_kernel<_Float16>, dim3((unsigned)blocks), dim3(ADAM_BLOCK), 0, s, t);
        }))
      return st;
  }
  return MNS_OK;
}

}  // namespace

// ====================================================================== C ABI

extern "C" {

int mns_workspace_bytes(int variant, const mns_tensor* G, const mns_ns_params* p,
                        int64_t max_batch_chunk, size_t* bytes) {
  if (!bytes) return MNS_ERR_ARG;
  if (variant != MNS_VARIANT_STANDARD && variant != MNS_VARIANT_GRAM) return MNS_ERR_ARG;
  if (int st = check_tensor(G, false)) return st;
  NsConf c;
  if (int st = check_params(p, G->dtype, &c, G, 1)) return st;
  const int64_t chunk = max_batch_chunk <= 0 ? G->batch : std::min(max_batch_chunk, G->batch);
  *bytes = plan(variant, geometry(G), c, chunk).total;
  return MNS_OK;
}

int muon_ns_batched(const mns_tensor* G, const mns_tensor* O, const mns_ns_params* p, void* ws,
                    size_t ws_bytes, int32_t* flags, void* stream) {
  return ns_entry(MNS_VARIANT_STANDARD, G, O, p, ws, ws_bytes, flags, stream);
}

int gram_ns_batched(const mns_tensor* G, const mns_tensor* O, const mns_ns_params* p, void* ws,
                    size_t ws_bytes, int32_t* flags, void* stream) {
  return ns_entry(MNS_VARIANT_GRAM, G, O, p, ws, ws_bytes, flags, stream);
}

int muon_step(const mns_tensor* W, const mns_tensor* G, const mns_tensor* M, const mns_tensor* U_out,
              const mns_step_params* sp, const mns_ns_params* p, void* ws, size_t ws_bytes,
              int32_t* flags, void* stream) {
  if (int st = check_step(W, G, M, U_out)) return st;
  if (int st = check_step_params(sp)) return st;
  NsConf c;
  if (int st = check_params(p, G->dtype, &c, G, 1)) return st;
  if (!ws) return MNS_ERR_WORKSPACE;
  Source src;
  FinalOut fo;
  step_io(W, G, M, U_out, sp, &src, &fo);
  return run_ns(sp->variant, src, fo, c, ws, ws_bytes, flags, reinterpret_cast<hipStream_t>(stream));
}

int muon_step_noalloc(const mns_tensor* W, const mns_tensor* G, const mns_tensor* M,
                      const mns_tensor* U_out, const mns_step_params* sp, const mns_ns_params* p,
                      int32_t* flags, void* stream) {
  if (int st = check_step(W, G, M, U_out)) return st;
  if (int st = check_step_params(sp)) return st;
  NsConf c;
  if (int st = check_params(p, G->dtype, &c, G, 1)) return st;
  const size_t cap = MNS_NOALLOC_SCRATCH_BYTES;
  if (pick_chunk(sp->variant, geometry(G), c, G->batch, cap) < 1) return MNS_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (int st = scratch_address(s, &ws)) return st;
  Source src;
  FinalOut fo;
  step_io(W, G, M, U_out, sp, &src, &fo);
  return run_ns(sp->variant, src, fo, c, ws, cap, flags, s);
}

int mns_workspace_bytes_grouped(int variant, int ngroups, const mns_tensor* G, const mns_ns_params* p,
                                size_t* bytes) {
  if (!bytes || !G) return MNS_ERR_ARG;
  if (variant != MNS_VARIANT_STANDARD && variant != MNS_VARIANT_GRAM) return MNS_ERR_ARG;
  if (ngroups < 1 || ngroups > MNS_MAXG) return MNS_ERR_ARG;
  for (int i = 0; i < ngroups; ++i) {
    if (int st = check_tensor(&G[i], false)) return st;
    if (G[i].dtype != G[0].dtype) return MNS_ERR_DTYPE;
  }
  NsConf c;
  if (int st = check_params(p, G[0].dtype, &c, G, ngroups)) return st;
  *bytes = grouped_bytes(variant, ngroups, G, c);
  return MNS_OK;
}

int muon_step_grouped(int ngroups, const mns_tensor* W, const mns_tensor* G, const mns_tensor* M,
                      const mns_tensor* U_out, const mns_step_params* sp, const mns_ns_params* p,
                      void* ws, size_t ws_bytes, int32_t* flags, void* stream) {
  if (ngroups < 1 || ngroups > MNS_MAXG || !W || !G || !M) return MNS_ERR_ARG;
  if (int st = check_step_params(sp)) return st;
  const mns_tensor* all[4 * MNS_MAXG];
  int na = 0;
  for (int i = 0; i < ngroups; ++i) {
    if (int st = check_step(&W[i], &G[i], &M[i], U_out ? &U_out[i] : nullptr)) return st;
    if (G[i].dtype != G[0].dtype) return MNS_ERR_DTYPE;
    all[na++] = &W[i];
    all[na++] = &G[i];
    all[na++] = &M[i];
    if (U_out) all[na++] = &U_out[i];
  }
  if (any_overlap(all, na)) return MNS_ERR_ARG;
  NsConf c;
  if (int st = check_params(p, G[0].dtype, &c, G, ngroups)) return st;
  if (!ws) return MNS_ERR_WORKSPACE;
  Source srcs[MNS_MAXG];
  FinalOut fos[MNS_MAXG];
  for (int i = 0; i < ngroups; ++i) step_io(&W[i], &G[i], &M[i], U_out ? &U_out[i] : nullptr, sp, &srcs[i], &fos[i]);
  return run_groups(sp->variant, ngroups, srcs, fos, c, ws, ws_bytes, flags, reinterpret_cast<hipStream_t>(stream));
}

static int ns_grouped(int variant, int ngroups, const mns_tensor* G, const mns_tensor* O,
                      const mns_ns_params* p, void* ws, size_t ws_bytes, int32_t* flags, void* stream) {
  if (ngroups < 1 || ngroups > MNS_MAXG || !G || !O) return MNS_ERR_ARG;
  const mns_tensor* all[2 * MNS_MAXG];
  int na = 0;
  for (int i = 0; i < ngroups; ++i) {
    if (int st = check_tensor(&G[i])) return st;
    if (int st = check_tensor(&O[i])) return st;
    if (!same_shape(&G[i], &O[i])) return MNS_ERR_SHAPE;
    if (O[i].dtype != G[i].dtype || G[i].dtype != G[0].dtype) return MNS_ERR_DTYPE;
    all[na++] = &O[i];
  }
  if (any_overlap(all, na)) return MNS_ERR_ARG;
  for (int i = 0; i < ngroups; ++i)
    for (int j = 0; j < ngroups; ++j)
      if (overlap(&G[i], &O[j])) return MNS_ERR_ARG;
  NsConf c;
  if (int st = check_params(p, G[0].dtype, &c, G, ngroups)) return st;
  if (!ws) return MNS_ERR_WORKSPACE;
  Source srcs[MNS_MAXG];
  FinalOut fos[MNS_MAXG];
  for (int i = 0; i < ngroups; ++i) {
    srcs[i].G = &G[i];
    fos[i].O = &O[i];
  }
  return run_groups(variant, ngroups, srcs, fos, c, ws, ws_bytes, flags, reinterpret_cast<hipStream_t>(stream));
}

int muon_ns_grouped(int ngroups, const mns_tensor* G, const mns_tensor* O, const mns_ns_params* p,
                    void* ws, size_t ws_bytes, int32_t* flags, void* stream) {
  return ns_grouped(MNS_VARIANT_STANDARD, ngroups, G, O, p, ws, ws_bytes, flags, stream);
}

int gram_ns_grouped(int ngroups, const mns_tensor* G, const mns_tensor* O, const mns_ns_params* p,
                    void* ws, size_t ws_bytes, int32_t* flags, void* stream) {
  return ns_grouped(MNS_VARIANT_GRAM, ngroups, G, O, p, ws, ws_bytes, flags, stream);
}

int gram_ns_trace(const mns_tensor* G, const mns_tensor* O, const mns_ns_params* p, void* ws,
                   size_t ws_bytes, float* trace, void* stream) {
  if (int st = check_tensor(G)) return st;
  if (int st = check_tensor(O)) return st;
  if (!same_shape(G, O)) return MNS_ERR_SHAPE;
  if (O->dtype != G->dtype) return MNS_ERR_DTYPE;
  if (overlap(G, O)) return MNS_ERR_ARG;
  if (!trace) return MNS_ERR_ARG;
  NsConf c;
  if (int st = check_params(p, G->dtype, &c, G, 1)) return st;
  if (c.steps < 2) return MNS_ERR_ARG;
  if (!ws) return MNS_ERR_WORKSPACE;
  mns_tensor g1 = *G, o1 = *O;
  g1.batch = 1;
  o1.batch = 1;
  Source src;
  src.G = &g1;
  FinalOut fo;
  fo.O = &o1;
  return run_ns(MNS_VARIANT_GRAM, src, fo, c, ws, ws_bytes, nullptr,
                reinterpret_cast<hipStream_t>(stream), trace);
}

int adamw_step(int ntensors, void* const* params, const void* const* grads, float* const* exp_avg,
               float* const* exp_avg_sq, const int64_t* numels, int32_t dtype,
               const mns_adamw_params* ap, void* stream) {
  if (ntensors < 1 || !params || !grads || !exp_avg || !exp_avg_sq || !numels || !ap) return MNS_ERR_ARG;
  if (!valid_dtype(dtype)) return MNS_ERR_DTYPE;
  const float hp[5] = {ap->lr, ap->beta1, ap->beta2, ap->eps, ap->weight_decay};
  for (float x : hp)
    if (!std::isfinite(x)) return MNS_ERR_ARG;
  if (ap->beta1 < 0.f || ap->beta1 >= 1.f || ap->beta2 < 0.f || ap->beta2 >= 1.f || ap->eps < 0.f) return MNS_ERR_ARG;
  if (ap->bias_correction != 0 && ap->bias_correction != 1) return MNS_ERR_ARG;
  if (ap->bias_correction && ap->step < 1) return MNS_ERR_ARG;
  // every buffer non-null (unless empty) and no two buffers overlapping
  std::vector<std::pair<uintptr_t, uintptr_t>> iv;
  const size_t es = (size_t)dtype_size(dtype);
  for (int i = 0; i < ntensors; ++i) {
    if (numels[i] < 0) return MNS_ERR_ARG;
    if (numels[i] == 0) continue;
    if (!params[i] || !grads[i] || !exp_avg[i] || !exp_avg_sq[i]) return MNS_ERR_ARG;
    const uintptr_t n = (uintptr_t)numels[i];
    iv.push_back({reinterpret_cast<uintptr_t>(params[i]), reinterpret_cast<uintptr_t>(params[i]) + n * es});
    iv.push_back({reinterpret_cast<uintptr_t>(grads[i]), reinterpret_cast<uintptr_t>(grads[i]) + n * es});
    iv.push_back({reinterpret_cast<uintptr_t>(exp_avg[i]), reinterpret_cast<uintptr_t>(exp_avg[i]) + n * 4});
    iv.push_back({reinterpret_cast<uintptr_t>(exp_avg_sq[i]), reinterpret_cast<uintptr_t>(exp_avg_sq[i]) + n * 4});
  }
  std::sort(iv.begin(), iv.end());
  for (size_t k = 1; k < iv.size(); ++k)
    if (iv[k].first < iv[k - 1].second) return MNS_ERR_ARG;
  return run_adamw(ntensors, params, grads, exp_avg, exp_avg_sq, numels, dtype, ap,
                   reinterpret_cast<hipStream_t>(stream));
}

const char* mns_status_string(int code) {
  switch (code) {
    case MNS_OK: return "ok";
    case MNS_ERR_ARG: return "invalid argument";
    case MNS_ERR_DTYPE: return "unsupported dtype or dtype combination";
    case MNS_ERR_SHAPE: return "invalid or mismatched shape";
    case MNS_ERR_WORKSPACE: return "workspace missing or too small";
    case MNS_ERR_HIP: return "HIP runtime error";
    case MNS_ERR_UNSUPPORTED: return "unsupported request";
    default: return "unknown status";
  }
}

int mns_last_hip_error(void) { return g_last_hip; }

int mns_version(void) { return 100; }

int mns_timing_enable(int on) {
  Timing& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  t.on = on != 0;
  return MNS_OK;
}

int mns_timing_reset(void) {
  Timing& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  for (auto& v : t.ev) {
    for (auto& pr : v) {
      t.pool.push_back(pr.first);
      t.pool.push_back(pr.second);
    }
    v.clear();
  }
  return MNS_OK;
}

int mns_timing_query(int kind, double* total_ms, int64_t* launches) {
  if (kind < 0 || kind >= NKINDS || !total_ms || !launches) return MNS_ERR_ARG;
  Timing& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  double tot = 0.0;
  for (auto& pr : t.ev[kind]) {
    hipError_t e = hipEventSynchronize(pr.second);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, pr.first, pr.second);
    if (e != hipSuccess) {
      g_last_hip = (int)e;
      return MNS_ERR_HIP;
    }
    tot += ms;
  }
  *total_ms = tot;
  *launches = (int64_t)t.ev[kind].size();
  return MNS_OK;
}

int mns_timing_kinds(void) { return NKINDS; }

const char* mns_kernel_kind_name(int kind) {
  return (kind >= 0 && kind < NKINDS) ? kKindNames[kind] : nullptr;
}

}  // extern "C"
