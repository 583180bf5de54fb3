// C ABI of libnmsparse: host-side validation and dispatch.  Every entry point checks
// its arguments completely before the first HIP call and then enqueues kernels on the
// caller's stream.  See include/nm.h for the contract of each call.
#include <hip/hip_runtime.h>

#include <mutex>

#include "nm.h"
#include "nm_launch.h"

namespace {

constexpr int kVersion = 100;  // 0.1.0

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool supported_m(int m) { return m == 4 || m == 8 || m == 16 || m == 32; }
// group widths the select / compact / scatter kernels also take (no bitmask)
inline bool select_only_m(int m) { return m == 6 || m == 10 || m == 12 || m == 14; }

inline bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  return !__builtin_mul_overflow(a, b, out);
}

// rows x ld matrix addressable (and no int64 overflow when scaled by 8 bytes)
inline bool span_ok(int64_t rows, int64_t ld) {
  int64_t e, b;
  return mul_ok(rows, ld, &e) && mul_ok(e, 8, &b);
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline nm_status hip_status(hipError_t e) { return e == hipSuccess ? NM_OK : NM_EHIP; }

__global__ void k_fill_zero_f32(float* y, int64_t rows, int64_t cols, int64_t ldy) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * cols) return;
  const int64_t r = i / cols, c = i - r * cols;
  y[r * ldy + c] = 0.f;
}

nm_status zero_output(float* y, int64_t rows, int64_t cols, int64_t ldy, hipStream_t s) {
  const int64_t n = rows * cols;
  if (n == 0) return NM_OK;
  k_fill_zero_f32<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(y, rows, cols, ldy);
  return hip_status(hipGetLastError());
}

// Common checks of a dense bf16 operand [rows][ld] covering k columns.  ld_mult: the
// leading dimension must be a multiple of this many elements (8 = 16-byte rows).
nm_status check_bf16(const void* p, int64_t rows, int64_t k, int64_t ld, bool required, int ld_mult = 8) {
  if (p == nullptr) return (required && rows > 0 && k > 0) ? NM_EINVAL : NM_OK;
  if (ld < k) return NM_ESHAPE;
  if (!span_ok(rows, ld)) return NM_ESHAPE;
  if (!aligned16(p) || (ld % ld_mult) != 0) return NM_EALIGN;
  return NM_OK;
}

// Row alignment the group kernels need: one group of m bf16 per lane, loaded in one
// piece of min(16, 2m) bytes.
inline int group_ld_mult(int m) { return select_only_m(m) ? 2 : (m < 8 ? m : 8); }


nm_status check_pattern(int64_t k, int n, int m) {
  if (!supported_m(m)) return (m >= 1 && n >= 1 && n <= m) ? NM_EUNSUPPORTED : NM_EINVAL;
  if (n < 1 || n > m) return NM_EINVAL;
  if (k < 0 || (k % m) != 0) return NM_ESHAPE;
  return NM_OK;
}

// check_pattern for the select-family calls: also the (2N-2):2N widths, when no bitmask
// is requested
nm_status check_select_pattern(int64_t k, int n, int m, bool mask) {
  if (!select_only_m(m)) return check_pattern(k, n, m);
  if (n < 1 || n > m) return NM_EINVAL;
  if (mask) return NM_EUNSUPPORTED;
  if (k < 0 || (k % m) != 0) return NM_ESHAPE;
  return NM_OK;
}

// The route hints of a call (nm.h); the size queries pass report = false so that they
// never write the caller's report.
nml::Route route_of(const nm_spmm_args* a, bool report) {
  nml::Route r{};
  r.flags = a->route;
  r.few_wpb = a->few_wpb; r.few_splits = a->few_splits; r.tile_wg = a->tile_wg;
  r.taken = report ? a->route_taken : nullptr;
  return r;
}

// Which activation route nm_spmm takes above the few-token range (the NM_ROUTE_ACT_*
// hints choose one; sx by default, fused when there is no workspace for S(X)):
//   fused: top-n selected inside the product kernel's X-tile loader;
//   mask:  a select pass writes the keep bitmask, the product applies it to X fragments;
//   sx:    a select pass writes S(X) to the workspace, the product streams it unchanged.
// Measured on gfx950, 8:16: at 8192 x 14336 x 4096 sx 90 + 767 us, mask 67 + 1091 us; the
// fused loader re-selects X once per output tile and is slower at every size (192 tokens
// on 4096 x 14336: 509 us, against 263 us for sx on the same register-staged kernel).
enum ActRoute { ROUTE_FUSED = 0, ROUTE_MASK = 1, ROUTE_SX = 2 };

ActRoute act_route(const nml::Route& r) {
  if (r.has(NM_ROUTE_ACT_FUSED)) return ROUTE_FUSED;
  if (r.has(NM_ROUTE_ACT_MASK)) return ROUTE_MASK;
  return ROUTE_SX;
}

// ----------------------------------------------------- no-allocation entry point ---
// The scratch of nm_spmm_noalloc: a file-scope device array, one copy per GPU, held by the
// library's code object until the process ends.  Host code never uses the array's name
// as an address (on the host it is only a stand-in for the symbol): each GPU's address is
// looked up once, with that GPU current, and kept below.


__device__ __align__(256) unsigned char scratch[NM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// This GPU's copy of the scratch array (null on failure, with the HIP error in *err).
void* scratch_for_current_device(hipError_t* err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  *err = g_scratch_err[dev];
  return g_scratch_ptr[dev];
}

int64_t mask_words(int64_t t, int64_t k) { return t * ((k + 31) / 32); }

// Token counts up to this go to the few-token kernels (decode shapes).
constexpr int64_t kFewMaxT = 128;

bool use_few(int64_t t, const nml::Route& r) { return t <= kFewMaxT && !r.has(NM_ROUTE_NO_FEW); }

// Above the few-token range, 256 x 256 output tiles that number under 256 leave CUs idle on
// the large-tile kernels (one workgroup per tile, each running the whole reduction).  Two
// remedies, chosen per call by large_plan:
//   split: the large-tile kernel with its reduction split in 2-4 K ranges (at most one
//     round of workgroups), when each range keeps enough K-steps to outweigh writing and
//     re-reading the partial tiles: 100 steps of 64 for the dense kernel, 32 for the
//     sparse kernel (whose steps take about twice as long);
//   mid: otherwise, under 128 tiles, the split-K 128-row tile kernel of the few-token
//     products, whose splits fill the chip.
// A second kernel sums the partial tiles (workspace) in split order.  Measured on gfx950
// (graph replays, cold weights, us, unsplit large-tile route -> plan):
//   8:16 S(X) x bf16 4096 x 14336: 192 tokens 263 -> 58 (mid), 512: 304 -> 96 (mid),
//     1024: 310 -> 144 (mid), 1536: 321 -> 200 (split), 2048: 261 -> 242 (split);
//   8:16 S(X) x bf16 14336 x 4096: 192: 87 -> 49 (mid), 512: 108 -> 88 (mid);
//   lowered 6:8 4096 x 4096: 256: 161 -> 36 (mid), 1024: 166 -> 71 (mid), 1536: 200 -> 105
//     (split), 2048: 126 -> 114 (split);
//   2:4 4096 x 14336: 1024 / 1536 / 2048 tokens split 119 / 165 / 187 (mid 133 / 233 / 245).
// The other choice, where measured, was slower: the dense 4096 x 14336 product at 1024
// tokens split in four 157 us, 4096 x 4096 at 2048 tokens split in two 100 us against 77,
// lowered 6:8 4096 x 4096 at 1024 tokens split in four (24 steps each) 83-85 us against 71.
// The NM_ROUTE_NO_FEW, NM_ROUTE_TILE_REGS and NM_ROUTE_TILE_LDS hints keep the unsplit
// large-tile kernels.
constexpr int64_t kMinSplitStepsDense = 100, kMinSplitStepsSparse = 32;

// Internal route bit (not in nm.h): no split of the large tiles.  The no-allocation entry
// point sets it when the split's partial tiles would not fit its buffer.
constexpr uint32_t kRouteNoLargeSplit = 1u << 31;

enum class Large { kTiles, kMid, kSplit, kHalf };
struct LargePlan {
  Large kind;
  int64_t splits;
};

// steps: the product's K-steps (64 positions; 128 for the fp8 sparse kernel)
LargePlan large_plan(int64_t t, int64_t o, int64_t steps, int64_t min_steps, const nml::Route& r) {
  if (t <= kFewMaxT || r.has(NM_ROUTE_NO_FEW) || r.has(NM_ROUTE_TILE_REGS) || r.has(NM_ROUTE_TILE_LDS))
    return {Large::kTiles, 1};
  const int64_t tiles = ((o + 255) / 256) * ((t + 255) / 256);
  const int64_t sp = tiles > 0 ? 256 / tiles : 1;
  if (sp >= 2 && sp <= 4 && steps / sp >= min_steps && !r.has(kRouteNoLargeSplit)) return {Large::kSplit, sp};
  return {tiles < 128 ? Large::kMid : Large::kTiles, 1};
}

// The dense kernel also has 256 x 128 tiles: where the plan would split and those tiles
// fill at least three quarters of one round of workgroups (and at most one), it takes
// them unsplit instead (half: no partial tiles, no second pass).  Measured on gfx950 in
// one process (8:16 S(X) x bf16 4096 x 14336, us): 1536 tokens 181 against 187 split,
// 2048 tokens 200 against 232 split.  The 2:4-family kernel keeps the split (2:4 4096 x
// 14336 at 1536 / 2048 tokens 152 / 172 split against 214 / 214 unsplit).
LargePlan dense_plan(const nml::GemmArgs& g) {
  const LargePlan p = large_plan(g.t, g.o, g.k / 64, kMinSplitStepsDense, g.route);
  if (p.kind == Large::kSplit) {
    const int64_t halves = ((g.o + 255) / 256) * ((g.t + 127) / 128);
    if (halves >= 192 && halves <= 256) return {Large::kHalf, 1};
  }
  return p;
}

// Dense weights on an activation operand that is already S(X) (PRO_NONE), above the
// few-token range, by the plan: the split large tiles, the split 128-row tiles, or the
// large-tile kernels (which also take every other prologue).
nm_status run_dense_large(const nml::GemmArgs& g, float* part, int64_t part_bytes, hipStream_t s) {
  if (g.prologue == nml::PRO_NONE) {
    const LargePlan p = dense_plan(g);
    if (p.kind == Large::kHalf && nml::gemm_lds_eligible(g, true)) return hip_status(nml::launch_gemm_lds(g, s));
    if (p.kind == Large::kSplit && nml::gemm_lds_eligible(g, true))
      return hip_status(nml::launch_gemm_lds_split(g, p.splits, part, part_bytes, s));
    if (p.kind == Large::kMid && nml::gemm_lds_small_eligible(g))
      return hip_status(nml::launch_gemm_lds_small(g, part, part_bytes, s));
  }
  return hip_status(nml::launch_gemm_dense(g, s));
}

// Partial-sum bytes a large-token dense call reserves in its workspace for the plan (the
// kernels' eligibility is checked at the call, so this may over-reserve).
int64_t dense_large_part_bytes(int64_t t, int64_t o, int64_t k, const nml::Route& r) {
  nml::GemmArgs g{};
  g.t = t; g.o = o; g.k = k; g.route = r;
  const LargePlan p = dense_plan(g);
  if (p.kind == Large::kSplit) return p.splits * t * o * 4;
  if (p.kind == Large::kMid) return nml::gemm_lds_small_part_bytes(g);
  return 0;
}

LargePlan sparse_plan(const nml::SparseArgs& sa) {
  return large_plan(sa.t, sa.o, sa.f8 ? sa.kc / 128 : (sa.kc + sa.kd) / 64, kMinSplitStepsSparse, sa.route);
}

// Splits of the plan for a large-token 2:4-family product on the direct-to-LDS kernel (1
// when the plan does not split or the kernel does not take the shape).
int64_t sparse_splits(const nml::SparseArgs& sa) {
  const LargePlan p = sparse_plan(sa);
  return p.kind == Large::kSplit && nml::gemm_lds_sp_eligible(sa, true) ? p.splits : 1;
}

// Large-token 2:4-family products on the direct-to-LDS kernel: by its size rule or a
// hint, or split by the plan.
bool sparse_lds_large(const nml::SparseArgs& sa) { return nml::gemm_sparse_uses_lds(sa) || sparse_splits(sa) > 1; }

inline int64_t align256(int64_t b) { return (b + 255) / 256 * 256; }

// Scratch slice [off, bytes) of a workspace, or null / 0 when the workspace ends before off.
inline float* ws_slice(void* ws, int64_t ws_bytes, int64_t off, int64_t* avail) {
  if (ws == nullptr || ws_bytes <= off) {
    *avail = 0;
    return nullptr;
  }
  *avail = ws_bytes - off;
  return reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + off);
}

// Few-token product with a dense weight on an activation operand that is already S(X)
// (g.prologue == PRO_NONE).  Up to 32 tokens the weight-streaming kernel; above that the
// split-K tile kernel, whose workgroups share each X slice through LDS across 128 weight
// rows.  Measured on gfx950 (bf16 W, 33-128 tokens): 4096 x 14336 at 128 tokens 40 vs
// 73 us, 14336 x 4096 at 64 tokens 32 vs 46 us; for weights under 2048 rows the
// streaming kernel stays ahead.  The NM_ROUTE_FEW_STREAM / NM_ROUTE_FEW_TILE hints force either.
bool few_use_tile(const nml::GemmArgs& g) {
  if (!nml::gemm_lds_small_eligible(g)) return false;
  if (g.route.has(NM_ROUTE_FEW_TILE)) return true;
  if (g.route.has(NM_ROUTE_FEW_STREAM)) return false;
  return g.t > 32 && g.o >= 2048;
}

nml::FewArgs few_dense_args(const nml::GemmArgs& g) {
  nml::FewArgs f{};
  f.nseg = 1;
  nml::FewSeg& sg = f.seg[0];
  sg.w = g.w; sg.ldw = g.ldw; sg.w_kind = g.w_fp8 ? nml::WK_FP8 : nml::WK_BF16;
  sg.x = g.x; sg.ldx = g.ldx; sg.loader = nml::XL_PLAIN; sg.ns = 2; sg.k = g.k;
  f.w_scale = g.w_scale; f.t = g.t; f.o = g.o; f.y = g.y; f.ldy = g.ldy; f.accumulate = g.accumulate;
  f.route = g.route;
  f.row_scale = g.row_scale; f.row_shift = g.row_shift; f.col_shift = g.col_shift;
  return f;
}

int64_t dense_few_part_bytes(const nml::GemmArgs& g) {
  return few_use_tile(g) ? nml::gemm_lds_small_part_bytes(g) : nml::few_partial_bytes(few_dense_args(g));
}

nm_status run_dense_few(const nml::GemmArgs& g, float* part, int64_t part_bytes, hipStream_t s) {
  if (few_use_tile(g)) return hip_status(nml::launch_gemm_lds_small(g, part, part_bytes, s));
  return hip_status(nml::launch_few(few_dense_args(g), part, part_bytes, s));
}

// 2:4 (W_COMPRESSED) or lowered (W_SLIDE) weights, few tokens
nml::FewArgs few_sparse_args(const nm_spmm_args* a, int64_t kc, int ns) {
  nml::FewArgs f{};
  f.nseg = 1;
  nml::FewSeg& sg = f.seg[0];
  sg.w = a->w; sg.w_meta = (const uint8_t*)a->w_meta; sg.w_kind = nml::WK_SP24;
  sg.x = (const uint16_t*)a->x; sg.ldx = a->ldx; sg.ns = ns;
  sg.loader = a->mode == NM_W_SLIDE ? nml::XL_LIFT : nml::XL_PLAIN; sg.k = kc;
  f.t = a->t; f.o = a->o; f.y = a->y; f.ldy = a->ldy; f.accumulate = a->accumulate;
  f.route = route_of(a, true);
  return f;
}

// Reduction length of the 2:4 operand of the W_* modes (K, or K' for lowered weights).
int64_t w_mode_kc(const nm_spmm_args* a) {
  if (a->mode == NM_W_SLIDE) return (a->k / (2 * a->ns)) * 4 * (a->ns - 1);
  return a->k;
}

// Row stride of a materialised lifted X (16-byte rows).
inline int64_t lift_ld(int64_t kp) { return (kp + 7) / 8 * 8; }

// Few-token products with a 2:4 weight operand (plain, lowered or hybrid): the split-K
// tile kernel, whose workgroups share each X slice through LDS across 128 weight rows,
// when its shape rules hold, above 32 tokens for weights of at least 2048 rows and above
// 16 tokens from 8192 rows (or from 2048 rows for lowered weights, whose lift the tile
// loads do); the streaming kernel otherwise.  Measured on gfx950: 6:8 lowered 4096 x
// 4096 at 128 tokens 30 vs 58 us, at 24 / 32 tokens 16.9 / 18.0 vs 20.0 / 22.3 us (tile
// against stream), 14336 x 4096 at 16 tokens 40 vs 56 us; 2:4 14336 x 4096 at 33 tokens
// 31 vs 38 us.  The NM_ROUTE_FEW_STREAM / NM_ROUTE_FEW_TILE hints force either.  Above
// the few-token range the same kernel takes the mid plan of large_plan.
bool sp_few_tile(const nml::SparseArgs& sa) {
  if (!nml::gemm_lds_sp_eligible(sa, true)) return false;
  if (sa.t > kFewMaxT) return sparse_plan(sa).kind == Large::kMid;   // above the few-token range
  if (sa.route.has(NM_ROUTE_FEW_TILE)) return true;
  if (sa.route.has(NM_ROUTE_FEW_STREAM)) return false;
  return (sa.t > 32 && sa.o >= 2048) || (sa.t > 16 && (sa.o >= 8192 || (sa.lift_dma && sa.o >= 2048)));
}

// Lowered weights on the direct-to-LDS tile kernels: the loads build the lifted X rows
// from the raw X (bf16 weights; the NM_ROUTE_LIFT_COPY hint lifts X into the workspace
// first instead).
bool w_lift_dma(const nm_spmm_args* a) {
  return a->mode == NM_W_SLIDE && a->w_dtype == NM_W_BF16 && !(a->route & NM_ROUTE_LIFT_COPY);
}

// The W_* modes as a tile-kernel call.  Lowered weights: the raw X, lifted by the tile
// loads, or (NM_ROUTE_LIFT_COPY) X lifted into a buffer of row stride lift_ld(kc)
// (pointer filled in by the caller).
nml::SparseArgs w_mode_sparse_args(const nm_spmm_args* a, int64_t kc, int ns, bool report) {
  nml::SparseArgs sa{};
  sa.route = route_of(a, report);
  sa.w_vals = (const uint16_t*)a->w; sa.w_meta = (const uint8_t*)a->w_meta; sa.kc = kc;
  sa.x = (const uint16_t*)a->x; sa.ldx = a->ldx; sa.ns = ns;
  sa.loader = nml::XL_PLAIN;
  if (w_lift_dma(a)) {
    sa.loader = nml::XL_LIFT;
    sa.lift_dma = 1;
  } else if (a->mode == NM_W_SLIDE) {
    sa.ldx = lift_ld(kc);
  }
  sa.t = a->t; sa.o = a->o; sa.y = a->y; sa.ldy = a->ldy; sa.accumulate = a->accumulate; sa.trans_out = 0;
  return sa;
}

// Workspace bytes of the few-token tile route of the W_* modes ([lifted X][partials]; 0
// when it needs none), or -1 when that route does not apply.
int64_t w_mode_tile_bytes(const nm_spmm_args* a, int64_t kc, int ns) {
  const nml::SparseArgs sa = w_mode_sparse_args(a, kc, ns, false);
  if (!sp_few_tile(sa)) return -1;
  const int64_t lift = (a->mode == NM_W_SLIDE && !sa.lift_dma) ? align256(a->t * lift_ld(kc) * 2) : 0;
  return lift + nml::gemm_lds_sp_small_part_bytes(sa);
}

// Large-token 2:4-family products on the direct-to-LDS kernel read a K-blocked copy of the
// weight positions (o * kc / 8 bytes) from the workspace at byte offset `off` when the
// workspace holds it (the NM_ROUTE_NO_META_BLOCK hint keeps the row-major positions).
bool meta_block_wanted(const nml::SparseArgs& sa) {
  if (sa.route.has(NM_ROUTE_NO_META_BLOCK)) return false;
  return sa.kc > 0 && sa.w_meta != nullptr && sparse_lds_large(sa);
}
int64_t meta_block_ws(const nml::SparseArgs& sa) {
  if (sa.route.has(NM_ROUTE_NO_META_BLOCK) || sa.kc <= 0 || !sparse_lds_large(sa)) return 0;
  return nml::meta_block_bytes(sa.o, sa.kc);
}
nm_status use_meta_block(nml::SparseArgs& sa, void* ws, int64_t ws_bytes, int64_t off, hipStream_t s) {
  if (ws == nullptr || !meta_block_wanted(sa) || ws_bytes < off + nml::meta_block_bytes(sa.o, sa.kc)) return NM_OK;
  uint8_t* blk = reinterpret_cast<uint8_t*>(ws) + off;
  if (nml::launch_meta_block(sa.w_meta, sa.o, sa.kc, sa.f8 ? 16 : 8, blk, s) != hipSuccess) return NM_EHIP;
  sa.w_meta_blk = blk;
  sa.route.note(NM_TAKEN_META_BLOCK);
  return NM_OK;
}

// fp8 x fp8 route of the W_* modes with fp8 weights: workspace [token codes][token
// scales][K-blocked positions][partial sums (few tokens)].  kc % 128 == 0.
struct W8A8Layout {
  int64_t xq, xs, meta, part, total;
};
W8A8Layout w8a8_layout(int64_t t, int64_t o, int64_t kc, int64_t part_bytes) {
  W8A8Layout L{};
  L.xq = 0;
  L.xs = align256(t * kc);
  L.meta = L.xs + align256(t * 4);
  L.part = L.meta + align256(nml::meta_block_bytes(o, kc));
  L.total = L.part + part_bytes;
  return L;
}
nml::SparseArgs w8a8_args(const nm_spmm_args* a, int64_t kc, const uint8_t* xq, const float* xs, bool report) {
  nml::SparseArgs sa{};
  sa.route = route_of(a, report);
  sa.w_vals = (const uint16_t*)a->w; sa.w_meta = (const uint8_t*)a->w_meta; sa.kc = kc;
  sa.x = (const uint16_t*)xq; sa.ldx = kc; sa.loader = nml::XL_PLAIN; sa.ns = 2;
  sa.t = a->t; sa.o = a->o; sa.y = a->y; sa.ldy = a->ldy; sa.accumulate = a->accumulate; sa.trans_out = 0;
  sa.f8 = 1; sa.x_scale = xs; sa.w_scale = a->w_scale;
  return sa;
}
// Up to 16 tokens (one token block) the product streams the e4m3 2:4 codes through the
// weight-streaming kernel (widened to bf16 after their LDS read, exactly, and multiplied
// on the bf16 sparse instruction with the lifted e4m3 X widened alike: the same products,
// summed in fp32 in another order), unless the NM_ROUTE_FEW_TILE hint asks for the split
// tile kernel on the fp8 instruction.
bool w8a8_stream(const nm_spmm_args* a, const nml::Route& r) {
  return use_few(a->t, r) && a->t <= 16 && !r.has(NM_ROUTE_FEW_TILE);
}
nml::FewArgs w8a8_few_args(const nm_spmm_args* a, int64_t kc, const uint8_t* xq, const float* xs,
                           const nml::Route& r) {
  nml::FewArgs f{};
  f.route = r;
  nml::FewSeg& sg = f.seg[f.nseg++];
  sg.w = a->w; sg.ldw = kc / 2; sg.w_meta = (const uint8_t*)a->w_meta; sg.w_kind = nml::WK_SP24F8;
  sg.x = (const uint16_t*)xq; sg.ldx = kc; sg.loader = nml::XL_F8; sg.ns = 2; sg.k = kc;
  f.w_scale = a->w_scale; f.row_scale = xs;
  f.t = a->t; f.o = a->o; f.y = a->y; f.ldy = a->ldy; f.accumulate = a->accumulate;
  return f;
}
int64_t w8a8_part_bytes(const nm_spmm_args* a, int64_t kc) {
  const nml::SparseArgs sa = w8a8_args(a, kc, nullptr, nullptr, false);
  if (w8a8_stream(a, sa.route)) return nml::few_partial_bytes(w8a8_few_args(a, kc, nullptr, nullptr, sa.route));
  if (use_few(a->t, sa.route)) return nml::gemm_lds_sp_small_part_bytes(sa);
  const LargePlan p = sparse_plan(sa);
  if (p.kind == Large::kMid) return nml::gemm_lds_sp_small_part_bytes(sa);
  return p.kind == Large::kSplit ? p.splits * a->t * a->o * 4 : 0;
}
int64_t w8a8_ws_bytes(const nm_spmm_args* a, int64_t kc) {
  return w8a8_layout(a->t, a->o, kc, w8a8_part_bytes(a, kc)).total;
}
nm_status w8a8_product(const nm_spmm_args* a, int64_t kc, int ns, hipStream_t s) {
  const W8A8Layout L = w8a8_layout(a->t, a->o, kc, w8a8_part_bytes(a, kc));
  if (a->workspace == nullptr || a->workspace_bytes < L.total) return NM_EINVAL;
  char* ws = reinterpret_cast<char*>(a->workspace);
  uint8_t* xq = reinterpret_cast<uint8_t*>(ws + L.xq);
  float* xs = reinterpret_cast<float*>(ws + L.xs);
  const int qns = a->mode == NM_W_SLIDE ? ns : 2;
  {
    // one token: the streaming kernel quantizes and lifts the row itself (no separate pass)
    const nml::Route r = route_of(a, true);
    if (w8a8_stream(a, r)) {
      nml::FewArgs f = w8a8_few_args(a, kc, nullptr, xs, r);
      f.seg[0].x = (const uint16_t*)a->x;
      f.q_ns = qns;
      if (nml::few_quant_in_kernel(f))
        return hip_status(nml::launch_few(f, reinterpret_cast<float*>(ws + L.part), L.total - L.part, s));
    }
  }
  hipError_t e = nml::launch_quant_lift(qns, (const uint16_t*)a->x, a->t, a->k, a->ldx, xq, kc, xs, s);
  if (e != hipSuccess) return NM_EHIP;
  nml::SparseArgs sa = w8a8_args(a, kc, xq, xs, true);
  sa.route.note(NM_TAKEN_QUANT | (a->mode == NM_W_SLIDE && ns > 2 ? NM_TAKEN_LIFT : 0u));
  if (w8a8_stream(a, sa.route))
    return hip_status(nml::launch_few(w8a8_few_args(a, kc, xq, xs, sa.route),
                                      reinterpret_cast<float*>(ws + L.part), L.total - L.part, s));
  // few tokens, or the mid plan: the split tile kernel reads the row-major positions (a
  // blocked copy would cost a launch of about the product's own length); above that the
  // blocked copy pays
  const LargePlan p = sparse_plan(sa);
  if (use_few(a->t, sa.route) || p.kind == Large::kMid)
    return hip_status(nml::launch_gemm_lds_sp_small(sa, reinterpret_cast<float*>(ws + L.part), L.total - L.part, s));
  uint8_t* blk = reinterpret_cast<uint8_t*>(ws + L.meta);
  if (nml::launch_meta_block(sa.w_meta, sa.o, kc, 16, blk, s) != hipSuccess) return NM_EHIP;
  sa.w_meta_blk = blk;
  sa.route.note(NM_TAKEN_META_BLOCK);
  if (p.kind == Large::kSplit)
    return hip_status(nml::launch_gemm_lds_sp_split(sa, p.splits, reinterpret_cast<float*>(ws + L.part),
                                                    L.total - L.part, s));
  return hip_status(nml::launch_gemm_lds_sp(sa, s));
}

// Large-token ACT_DYNAMIC with fp8 weights: bytes of a bf16 copy of the weights in the
// workspace (after the S(X) staging) for the direct-to-LDS product kernel.
// Only when the codes cannot go to LDS directly (rows not 16-byte multiples), or under
// the NM_ROUTE_FP8_WIDEN hint.
int64_t fp8_widen_bytes(const nm_spmm_args* a) {
  const nml::Route r = route_of(a, false);
  if (a->mode != NM_ACT_DYNAMIC || a->pts != 0 || a->w_dtype != NM_W_FP8E4M3 || use_few(a->t, r)) return 0;
  if (a->k % 64 != 0 || a->t < 512) return 0;
  if (!r.has(NM_ROUTE_FP8_WIDEN) && a->ldw % 16 == 0) return 0;
  return a->o * a->k * 2;
}

// Bytes of S(X) / decompressed-X staging at the start of nm_spmm's workspace.  With the
// activation mitigations: [S(x~)][mu [t]][alpha [t]].
int64_t spmm_stage_bytes(const nm_spmm_args* a) {
  if (a->mode == NM_ACT_DYNAMIC && a->pts != 0) return align256(a->t * a->k * 2) + 2 * align256(a->t * 4);
  // also holds the 2:4 compressed X; 2-32 tokens may stage S(X) in whole 16-token blocks
  if (a->mode == NM_ACT_DYNAMIC) return (a->t >= 2 && a->t <= 32 ? (a->t + 15) / 16 * 16 : a->t) * a->k * 2 + 64;
  if (a->mode == NM_ACT_COMPRESSED) return a->t * a->k * 2;
  return 0;
}

// Hybrid: column-permuted X staging [t][ldp], dense region at column off1.
inline int64_t hybrid_off1(int64_t k_s) { return (k_s + 7) / 8 * 8; }
inline int64_t hybrid_ldp(int64_t k_s, int64_t k_d) { return hybrid_off1(k_s) + (k_d + 7) / 8 * 8; }

nml::FewArgs few_hybrid_args(const uint16_t* x, int64_t ldx, int64_t dbase, int64_t t, int64_t k_s, int64_t k_d,
                             const void* ws_values, const void* ws_meta, const void* wd, int64_t ldwd, int64_t o,
                             float* y, int64_t ldy, int accumulate, const nml::Route& r) {
  nml::FewArgs f{};
  f.route = r;
  if (k_s > 0) {
    nml::FewSeg& sg = f.seg[f.nseg++];
    sg.w = ws_values; sg.w_meta = (const uint8_t*)ws_meta; sg.w_kind = nml::WK_SP24;
    sg.x = x; sg.ldx = ldx; sg.loader = nml::XL_PLAIN; sg.ns = 2; sg.k = k_s;
  }
  if (k_d > 0) {
    nml::FewSeg& sg = f.seg[f.nseg++];
    sg.w = wd; sg.ldw = ldwd; sg.w_kind = nml::WK_BF16;
    sg.x = x + dbase; sg.ldx = ldx; sg.loader = nml::XL_PLAIN; sg.ns = 2; sg.k = k_d;
  }
  f.t = t; f.o = o; f.y = y; f.ldy = ldy; f.accumulate = accumulate;
  return f;
}

nml::SparseArgs hybrid_sparse_args(const uint16_t* x, int64_t ldx, int64_t dbase, int64_t t, int64_t k_s,
                                   int64_t k_d, const void* ws_values, const void* ws_meta, const void* wd,
                                   int64_t ldwd, int64_t o, float* y, int64_t ldy, int accumulate,
                                   const nml::Route& r) {
  nml::SparseArgs sa{};
  sa.route = r;
  sa.w_vals = (const uint16_t*)ws_values; sa.w_meta = (const uint8_t*)ws_meta; sa.kc = k_s;
  sa.x = x; sa.ldx = ldx; sa.loader = nml::XL_PLAIN;
  sa.t = t; sa.o = o;
  sa.wd = (const uint16_t*)wd; sa.ldwd = ldwd; sa.kd = k_d; sa.dbase = dbase;
  sa.y = y; sa.ldy = ldy; sa.accumulate = accumulate; sa.trans_out = 0;
  return sa;
}

}  // namespace

extern "C" {

const char* nm_status_str(nm_status s) {
  switch (s) {
    case NM_OK: return "NM_OK";
    case NM_EINVAL: return "NM_EINVAL: invalid argument";
    case NM_ESHAPE: return "NM_ESHAPE: inconsistent sizes";
    case NM_EALIGN: return "NM_EALIGN: misaligned pointer or leading dimension";
    case NM_EUNSUPPORTED: return "NM_EUNSUPPORTED: valid but not implemented";
    case NM_EHIP: return "NM_EHIP: HIP runtime error";
    case NM_ESCRATCH: return "NM_ESCRATCH: needs more scratch than nm_spmm_noalloc holds";
  }
  return "NM_?: unknown status";
}

int nm_version(void) { return kVersion; }

nm_status nm_sparsify(const void* x, int64_t rows, int64_t k, int64_t ldx, int n, int m, void* y,
                      int64_t ldy, uint32_t* mask, void* stream) {
  nm_status st = check_select_pattern(k, n, m, mask != nullptr);
  if (st) return st;
  if (rows < 0) return NM_ESHAPE;
  if (y == nullptr && mask == nullptr) return NM_EINVAL;
  if ((st = check_bf16(x, rows, k, ldx, true, group_ld_mult(m)))) return st;
  if ((st = check_bf16(y, rows, k, ldy, false, group_ld_mult(m)))) return st;
  if (mask != nullptr && !aligned16(mask)) return NM_EALIGN;
  if (rows == 0 || k == 0) return NM_OK;
  return hip_status(nml::launch_select(m, (const uint16_t*)x, rows, k, ldx, n, (uint16_t*)y, ldy, mask,
                                       nullptr, nullptr, 0, as_stream(stream)));
}

nm_status nm_sparsify_scored(const void* x, int64_t rows, int64_t k, int64_t ldx, int n, int m,
                             const float* col_score, nm_score mode, void* y, int64_t ldy, uint32_t* mask,
                             void* stream) {
  if (m != 4 && m != 8 && m != 16 && m != 32)
    return (m >= 1 && n >= 1 && n <= m) ? NM_EUNSUPPORTED : NM_EINVAL;
  nm_status st = check_pattern(k, n, m);
  if (st) return st;
  if (rows < 0) return NM_ESHAPE;
  if (mode != NM_SCORE_ACT_WEIGHTED && mode != NM_SCORE_WEIGHT) return NM_EINVAL;
  if (y == nullptr && mask == nullptr) return NM_EINVAL;
  if (col_score == nullptr && k > 0) return NM_EINVAL;
  if ((st = check_bf16(x, rows, k, ldx, true, group_ld_mult(m)))) return st;
  if ((st = check_bf16(y, rows, k, ldy, false, group_ld_mult(m)))) return st;
  if ((mask != nullptr && !aligned16(mask)) || (col_score != nullptr && !aligned16(col_score))) return NM_EALIGN;
  if (rows == 0 || k == 0) return NM_OK;
  return hip_status(nml::launch_select_scored(m, (const uint16_t*)x, rows, k, ldx, n, col_score,
                                              mode == NM_SCORE_ACT_WEIGHTED ? 1 : 0, (uint16_t*)y, ldy, mask,
                                              as_stream(stream)));
}

nm_status nm_sparsify_pts(const void* x, int64_t rows, int64_t k, int64_t ldx, int n, int m, int pts,
                          const float* shift, void* y, int64_t ldy, uint32_t* mask, float* row_shift,
                          float* row_scale, void* stream) {
  nm_status st = check_pattern(k, n, m);
  if (st) return st;
  if (rows < 0) return NM_ESHAPE;
  if ((pts & ~(NM_PTS_DYNAMIC | NM_PTS_STATIC | NM_PTS_VAR)) != 0) return NM_EINVAL;
  if ((pts & NM_PTS_DYNAMIC) && (pts & NM_PTS_STATIC)) return NM_EINVAL;
  if ((pts & NM_PTS_STATIC) && shift == nullptr && k > 0) return NM_EINVAL;
  if ((pts & NM_PTS_VAR) && row_scale == nullptr && rows > 0) return NM_EINVAL;
  if (y == nullptr && rows > 0 && k > 0) return NM_EINVAL;
  if (k % 8 != 0 || k > 65536) return NM_ESHAPE;
  if ((st = check_bf16(x, rows, k, ldx, true))) return st;
  if ((st = check_bf16(y, rows, k, ldy, true))) return st;
  if (!aligned16(mask) || !aligned16(shift) || !aligned16(row_shift) || !aligned16(row_scale)) return NM_EALIGN;
  if (rows == 0 || k == 0) return NM_OK;
  if (rows > 0x7FFFFFFF) return NM_ESHAPE;
  const bool dyn = (pts & NM_PTS_DYNAMIC) != 0;
  return hip_status(nml::launch_select_pts(m, (const uint16_t*)x, rows, k, ldx, n, dyn ? 1 : 0,
                                           (pts & NM_PTS_STATIC) ? shift : nullptr, (pts & NM_PTS_VAR) ? 1 : 0,
                                           (uint16_t*)y, ldy, mask, dyn ? row_shift : nullptr,
                                           (pts & NM_PTS_VAR) ? row_scale : nullptr, as_stream(stream)));
}

nm_status nm_weight_sums(const void* w, int64_t o, int64_t k, int64_t ldw, int w_dtype, const float* w_scale,
                         const float* shift, float* out, void* stream) {
  if (o < 0 || k < 0) return NM_ESHAPE;
  if (w_dtype != NM_W_BF16 && w_dtype != NM_W_FP8E4M3) return NM_EINVAL;
  nm_status st;
  if (w_dtype == NM_W_BF16) {
    if ((st = check_bf16(w, o, k, ldw, true, 1))) return st;
  } else {
    if (w == nullptr && o > 0 && k > 0) return NM_EINVAL;
    if (ldw < k || !span_ok(o, ldw)) return NM_ESHAPE;
    if (w_scale == nullptr && o > 0) return NM_EINVAL;
  }
  if (out == nullptr && o > 0) return NM_EINVAL;
  if (!aligned16(w) || !aligned16(w_scale) || !aligned16(shift) || !aligned16(out)) return NM_EALIGN;
  if (o == 0) return NM_OK;
  return hip_status(nml::launch_weight_sums(w, o, k, ldw, w_dtype == NM_W_FP8E4M3 ? 1 : 0,
                                            w_dtype == NM_W_FP8E4M3 ? w_scale : nullptr, shift, out,
                                            as_stream(stream)));
}

nm_status nm_compress(const void* x, int64_t rows, int64_t k, int64_t ldx, int n, int m, void* values,
                      void* meta, nm_meta fmt, uint32_t* mask, void* stream) {
  nm_status st = check_select_pattern(k, n, m, mask != nullptr);
  if (st) return st;
  if (rows < 0) return NM_ESHAPE;
  if (fmt != NM_META_U8 && fmt != NM_META_2BIT) return NM_EINVAL;
  if (fmt == NM_META_2BIT && !(n == 2 && m == 4)) return NM_EINVAL;
  if ((st = check_bf16(x, rows, k, ldx, true, group_ld_mult(m)))) return st;
  if (rows > 0 && k > 0 && (values == nullptr || meta == nullptr)) return NM_EINVAL;
  if (!span_ok(rows, k)) return NM_ESHAPE;
  if ((values && !aligned16(values)) || (meta && !aligned16(meta)) || (mask && !aligned16(mask)))
    return NM_EALIGN;
  if (rows == 0 || k == 0) return NM_OK;
  return hip_status(nml::launch_select(m, (const uint16_t*)x, rows, k, ldx, n, nullptr, 0, mask,
                                       (uint16_t*)values, (uint8_t*)meta, fmt == NM_META_2BIT ? 1 : 0,
                                       as_stream(stream)));
}

nm_status nm_decompress(const void* values, const void* meta, nm_meta fmt, int64_t rows, int64_t k, int n,
                        int m, void* y, int64_t ldy, void* stream) {
  nm_status st = check_select_pattern(k, n, m, false);
  if (st) return st;
  if (rows < 0) return NM_ESHAPE;
  if (fmt != NM_META_U8 && fmt != NM_META_2BIT) return NM_EINVAL;
  if (fmt == NM_META_2BIT && !(n == 2 && m == 4)) return NM_EINVAL;
  if (rows > 0 && k > 0 && (values == nullptr || meta == nullptr)) return NM_EINVAL;
  if ((st = check_bf16(y, rows, k, ldy, true, group_ld_mult(m)))) return st;
  if (!span_ok(rows, k)) return NM_ESHAPE;
  if ((values && !aligned16(values)) || (meta && !aligned16(meta))) return NM_EALIGN;
  if (rows == 0 || k == 0) return NM_OK;
  return hip_status(nml::launch_decompress(m, (const uint16_t*)values, (const uint8_t*)meta,
                                           fmt == NM_META_2BIT ? 1 : 0, rows, k, n, (uint16_t*)y, ldy,
                                           as_stream(stream)));
}

nm_status nm_lower_slide(const void* values, const uint8_t* idx, int64_t rows, int64_t k, int ns,
                         void* values_out, void* meta_out, nm_meta fmt, void* stream) {
  if (ns < 2 || ns > 8) return (ns > 8) ? NM_EUNSUPPORTED : NM_EINVAL;
  if (fmt != NM_META_U8 && fmt != NM_META_2BIT) return NM_EINVAL;
  if (rows < 0 || k < 0 || (k % (2 * ns)) != 0) return NM_ESHAPE;
  if (!span_ok(rows, 2 * k)) return NM_ESHAPE;
  if (rows > 0 && k > 0 && (!values || !idx || !values_out || !meta_out)) return NM_EINVAL;
  if ((values && !aligned16(values)) || (idx && !aligned16(idx)) || (values_out && !aligned16(values_out)) ||
      (meta_out && !aligned16(meta_out)))
    return NM_EALIGN;
  if (rows == 0 || k == 0) return NM_OK;
  return hip_status(nml::launch_lower_slide(ns, (const uint16_t*)values, idx, rows, k, (uint16_t*)values_out,
                                            (uint8_t*)meta_out, fmt == NM_META_2BIT ? 1 : 0,
                                            as_stream(stream)));
}

nm_status nm_slide_lift(const void* x, int64_t t, int64_t k, int64_t ldx, int ns, void* x_out, int64_t ldo,
                        void* stream) {
  if (ns < 2 || ns > 8) return (ns > 8) ? NM_EUNSUPPORTED : NM_EINVAL;
  if (t < 0 || k < 0 || (k % (2 * ns)) != 0) return NM_ESHAPE;
  const int64_t kp = (k / (2 * ns)) * 4 * (ns - 1);
  nm_status st;   // element-wise kernel: any leading dimension
  if ((st = check_bf16(x, t, k, ldx, true, 1))) return st;
  if ((st = check_bf16(x_out, t, kp, ldo, true, 1))) return st;
  if (t == 0 || k == 0) return NM_OK;
  return hip_status(nml::launch_lift(ns, (const uint16_t*)x, t, k, ldx, (uint16_t*)x_out, ldo, as_stream(stream)));
}

nm_status nm_quant_lift(const void* x, int64_t t, int64_t k, int64_t ldx, int ns, void* xq, int64_t ldq, float* xs,
                        void* stream) {
  if (ns < 2 || ns > 8) return (ns > 8) ? NM_EUNSUPPORTED : NM_EINVAL;
  if (t < 0 || k < 0 || (k % (2 * ns)) != 0) return NM_ESHAPE;
  const int64_t kp = (k / (2 * ns)) * 4 * (ns - 1);
  nm_status st;
  if ((st = check_bf16(x, t, k, ldx, true, 1))) return st;
  if (ldq < kp || !span_ok(t, ldq)) return NM_ESHAPE;
  if ((ldq % 16) != 0) return NM_EALIGN;
  if (t > 0 && (xq == nullptr || xs == nullptr)) return NM_EINVAL;
  if ((xq && !aligned16(xq)) || (xs && !aligned16(xs))) return NM_EALIGN;
  if (t == 0) return NM_OK;
  return hip_status(nml::launch_quant_lift(ns, (const uint16_t*)x, t, k, ldx, (uint8_t*)xq, ldq, xs,
                                           as_stream(stream)));
}

// Single-token route over K-major weights (reads only the selected K-rows).
bool gather1_route(const nm_spmm_args* a) {
  return a->mode == NM_ACT_DYNAMIC && a->pts == 0 && a->t == 1 && a->w_kmajor != nullptr && a->w_dtype == NM_W_BF16 &&
         a->w_scale == nullptr && a->o > 0 && a->k > 0 && (a->o % 8) == 0 && supported_m(a->m);
}

int64_t nm_spmm_workspace_size(const nm_spmm_args* a) {
  if (a == nullptr || a->t < 0 || a->o < 0 || a->k < 0) return 0;
  if ((a->mode == NM_W_COMPRESSED || a->mode == NM_W_SLIDE) && a->w_dtype == NM_W_FP8E4M3) {
    if (a->mode == NM_W_SLIDE && (a->ns < 2 || a->ns > 8 || a->k % (2 * a->ns))) return 0;
    const int64_t kc = w_mode_kc(a);
    return (a->t > 0 && a->o > 0 && kc > 0 && kc % 128 == 0) ? w8a8_ws_bytes(a, kc) : 0;
  }
  if (gather1_route(a)) return nml::gather1_part_bytes(a->k, a->o, a->m);
  const nml::Route r = route_of(a, false);
  const int64_t stage = spmm_stage_bytes(a);
  int64_t part = 0;
  if (use_few(a->t, r) && a->t > 0 && a->o > 0 && a->k > 0) {
    if (a->mode == NM_W_COMPRESSED || a->mode == NM_W_SLIDE) {
      if (a->mode == NM_W_SLIDE && (a->ns < 2 || a->ns > 8 || a->k % (2 * a->ns))) return 0;
      const int ns = a->mode == NM_W_SLIDE ? a->ns : 2;
      const int64_t tile = w_mode_tile_bytes(a, w_mode_kc(a), ns);
      if (tile >= 0) return tile;
      nml::FewArgs f = few_sparse_args(a, w_mode_kc(a), ns);
      f.route = r;
      part = nml::few_partial_bytes(f);
    } else if (a->mode == NM_ACT_DYNAMIC || a->mode == NM_ACT_COMPRESSED ||
               (a->mode == NM_ACT_MASKED && a->x_meta == nullptr)) {
      nml::GemmArgs g{};
      g.w = a->w; g.ldw = a->ldw; g.w_fp8 = a->w_dtype == NM_W_FP8E4M3 ? 1 : 0; g.w_scale = a->w_scale;
      g.t = a->t; g.o = a->o; g.k = a->k; g.prologue = nml::PRO_NONE; g.route = r;
      g.ldx = a->mode == NM_ACT_MASKED ? a->ldx : a->k;
      part = dense_few_part_bytes(g);
    }
  }
  if (part > 0) return align256(stage) + part;
  if ((a->mode == NM_W_SLIDE || a->mode == NM_W_COMPRESSED) && !use_few(a->t, r) && a->t > 0 && a->o > 0) {
    // large-token product: [lifted X (lowered weights)][K-blocked positions]
    if (a->mode == NM_W_SLIDE && (a->ns < 2 || a->ns > 8 || a->k % (2 * a->ns))) return 0;
    if (a->mode == NM_W_COMPRESSED && a->k % 4) return 0;
    const int64_t kc = w_mode_kc(a);
    if (a->t > kFewMaxT) {
      // the split tile kernel when the large tiles would not fill the chip
      const int64_t tile = w_mode_tile_bytes(a, kc, a->mode == NM_W_SLIDE ? a->ns : 2);
      if (tile >= 0) return tile;
    }
    nml::SparseArgs sa = w_mode_sparse_args(a, kc, a->mode == NM_W_SLIDE ? a->ns : 2, false);
    // [lifted X][K-blocked positions][partial sums of the split large tiles]; a lifted copy
    // of X only where the tile loads do not lift it themselves
    const bool lifted_loads = sa.lift_dma && sparse_lds_large(sa);
    int64_t lift = 0;
    if (a->mode == NM_W_SLIDE && !lifted_loads) {
      lift = align256(a->t * lift_ld(kc) * 2);
      sa.loader = nml::XL_PLAIN; sa.lift_dma = 0; sa.ldx = lift_ld(kc);   // the kernel then reads the copy
    }
    const int64_t mb = meta_block_ws(sa), sp = sparse_splits(sa);
    return lift + align256(mb) + (sp > 1 ? sp * a->t * a->o * 4 : 0);
  }
  const int64_t widen = fp8_widen_bytes(a);
  if (a->mode == NM_ACT_DYNAMIC || a->mode == NM_ACT_COMPRESSED || (a->mode == NM_ACT_MASKED && a->x_meta == nullptr)) {
    // [staging][widened W][partial sums of the split tiles]
    const int64_t part_l = dense_large_part_bytes(a->t, a->o, a->k, r);
    if (part_l > 0) return align256(stage) + (widen > 0 ? align256(widen) : 0) + part_l;
  }
  return widen > 0 ? align256(stage) + widen : stage;
}

}  // extern "C"

namespace {

// nm_spmm's body.  noalloc: the call brings no workspace (NM_EINVAL if it does); after the
// arguments are validated, the library's scratch buffer on the current GPU becomes the
// workspace (NM_ESCRATCH if the preferred route needs more).
nm_status spmm_impl(const nm_spmm_args* a, void* stream, bool noalloc) {
  if (a == nullptr) return NM_EINVAL;
  if (noalloc && (a->workspace != nullptr || a->workspace_bytes != 0)) return NM_EINVAL;
  nm_spmm_args local;
  // called where validation is complete, before the first HIP call
  auto bind_scratch = [&]() -> nm_status {
    if (!noalloc) return NM_OK;
    local = *a;
    int64_t need = nm_spmm_workspace_size(&local);
    if (need > NM_NOALLOC_SCRATCH_BYTES) {
      // without the split of the large tiles (whose partial tiles may not fit the buffer)
      local.route |= kRouteNoLargeSplit;
      need = nm_spmm_workspace_size(&local);
      if (need > NM_NOALLOC_SCRATCH_BYTES) return NM_ESCRATCH;
    }
    if (need > 0) {
      hipError_t e = hipSuccess;
      void* p = scratch_for_current_device(&e);
      if (p == nullptr) return NM_EHIP;
      local.workspace = p;
      local.workspace_bytes = need;
    }
    a = &local;
    return NM_OK;
  };
  const hipStream_t s = as_stream(stream);
  const int64_t T = a->t, O = a->o, K = a->k;
  if (T < 0 || O < 0 || K < 0) return NM_ESHAPE;
  if (a->accumulate != 0 && a->accumulate != 1) return NM_EINVAL;
  if (T > 0 && O > 0 && a->y == nullptr) return NM_EINVAL;
  if (a->y != nullptr) {
    if (a->ldy < O || !span_ok(T, a->ldy)) return NM_ESHAPE;
    if (!aligned16(a->y)) return NM_EALIGN;
  }
  // activation mitigations and output terms (ACT_* modes only)
  const bool epi_in = a->row_scale != nullptr || a->row_shift != nullptr || a->col_shift != nullptr;
  if (a->pts != 0 || epi_in) {
    if (a->mode == NM_W_COMPRESSED || a->mode == NM_W_SLIDE) return NM_EUNSUPPORTED;
    if ((a->pts & ~(NM_PTS_DYNAMIC | NM_PTS_STATIC | NM_PTS_VAR)) != 0) return NM_EINVAL;
    if ((a->pts & NM_PTS_DYNAMIC) && (a->pts & NM_PTS_STATIC)) return NM_EINVAL;
    if (a->pts != 0 && a->mode != NM_ACT_DYNAMIC) return NM_EINVAL;
    if (a->mode == NM_ACT_DYNAMIC && (a->row_scale != nullptr || a->row_shift != nullptr)) return NM_EINVAL;
    const bool shifted = (a->pts & (NM_PTS_DYNAMIC | NM_PTS_STATIC)) != 0;
    if (a->mode == NM_ACT_DYNAMIC && shifted != (a->col_shift != nullptr)) return NM_EINVAL;
    if ((a->pts & NM_PTS_STATIC) && a->pts_shift == nullptr && K > 0) return NM_EINVAL;
    if (a->row_shift != nullptr && a->col_shift == nullptr) return NM_EINVAL;
    if (!aligned16(a->pts_shift) || !aligned16(a->col_shift) || !aligned16(a->row_scale) ||
        !aligned16(a->row_shift))
      return NM_EALIGN;
    if (a->pts != 0 && (K % 8 != 0 || K > 65536)) return NM_ESHAPE;
  }
  nm_status st;
  switch (a->mode) {
    case NM_ACT_DYNAMIC:
    case NM_ACT_MASKED:
    case NM_ACT_COMPRESSED: {
      if ((st = check_pattern(K, a->n, a->m))) return st;
      if (a->w_dtype != NM_W_BF16 && a->w_dtype != NM_W_FP8E4M3) return NM_EINVAL;
      const bool fp8 = a->w_dtype == NM_W_FP8E4M3;
      if (fp8) {
        if (a->w == nullptr && O > 0 && K > 0) return NM_EINVAL;
        if (a->ldw < K || !span_ok(O, a->ldw)) return NM_ESHAPE;
        if ((a->w && !aligned16(a->w)) || (a->ldw % 16) != 0) return NM_EALIGN;
        if (a->w_scale == nullptr && O > 0) return NM_EINVAL;
      } else {
        if ((st = check_bf16(a->w, O, K, a->ldw, true))) return st;
      }
      if (a->w_scale != nullptr && !aligned16(a->w_scale)) return NM_EALIGN;
      if (a->mode == NM_ACT_DYNAMIC || a->mode == NM_ACT_MASKED) {
        if ((st = check_bf16(a->x, T, K, a->ldx, true))) return st;
        if (a->mode == NM_ACT_MASKED && a->x_meta != nullptr && !aligned16(a->x_meta)) return NM_EALIGN;
      } else {
        if (a->x_meta_fmt != NM_META_U8 && a->x_meta_fmt != NM_META_2BIT) return NM_EINVAL;
        if (a->x_meta_fmt == NM_META_2BIT && !(a->n == 2 && a->m == 4)) return NM_EINVAL;
        if (T > 0 && K > 0 && (a->x == nullptr || a->x_meta == nullptr)) return NM_EINVAL;
        if ((a->x && !aligned16(a->x)) || (a->x_meta && !aligned16(a->x_meta))) return NM_EALIGN;
      }
      if (a->x_mask_out != nullptr && !aligned16(a->x_mask_out)) return NM_EALIGN;
      if (a->workspace != nullptr && !aligned16(a->workspace)) return NM_EALIGN;
      if (a->w_kmajor != nullptr && !aligned16(a->w_kmajor)) return NM_EALIGN;
      if ((st = bind_scratch())) return st;
      if (T == 0 || O == 0) return NM_OK;
      if (K == 0) return a->accumulate ? NM_OK : zero_output(a->y, T, O, a->ldy, s);

      const nml::Route R = route_of(a, true);
      nml::GemmArgs g{};
      g.w = a->w; g.ldw = a->ldw; g.w_fp8 = fp8 ? 1 : 0; g.w_scale = a->w_scale;
      g.n = a->n; g.m = a->m; g.t = T; g.o = O; g.k = K;
      g.y = a->y; g.ldy = a->ldy; g.accumulate = a->accumulate; g.route = R;
      g.row_scale = a->row_scale; g.row_shift = a->row_shift; g.col_shift = a->col_shift;
      // workspace: [S(X) or decompressed X staging][few-token partial sums]
      const int64_t stage = spmm_stage_bytes(a);
      const bool have_ws = a->workspace != nullptr && a->workspace_bytes >= stage;
      int64_t part_avail = 0;
      float* part = ws_slice(a->workspace, a->workspace_bytes, stage > 0 ? align256(stage) : 0, &part_avail);

      if (a->mode == NM_ACT_COMPRESSED) {
        if (a->n == 2 && a->m == 4 && a->x_meta_fmt == NM_META_2BIT && !fp8 && a->w_scale == nullptr && !epi_in) {
          // 2:4 activations: X is the sparse operand of the sparse matrix instruction
          nml::SparseArgs sa{};
          sa.w_vals = (const uint16_t*)a->x; sa.w_meta = (const uint8_t*)a->x_meta; sa.kc = K;
          sa.x = (const uint16_t*)a->w; sa.ldx = a->ldw; sa.loader = nml::XL_PLAIN;
          sa.t = O; sa.o = T; sa.y = a->y; sa.ldy = a->ldy; sa.accumulate = a->accumulate; sa.trans_out = 1;
          sa.route = R;
          return hip_status(nml::launch_gemm_sparse(sa, s));
        }
        if (!have_ws) return NM_EINVAL;   // decompressed X needs the workspace
        uint16_t* xd = (uint16_t*)a->workspace;
        hipError_t e = nml::launch_decompress(a->m, (const uint16_t*)a->x, (const uint8_t*)a->x_meta,
                                              a->x_meta_fmt == NM_META_2BIT, T, K, a->n, xd, K, s);
        if (e != hipSuccess) return NM_EHIP;
        R.note(NM_TAKEN_DECOMPRESS);
        g.x = xd; g.ldx = K; g.prologue = nml::PRO_NONE;
        if (use_few(T, R)) return run_dense_few(g, part, part_avail, s);
        return run_dense_large(g, part, part_avail, s);
      }

      g.x = (const uint16_t*)a->x; g.ldx = a->ldx;
      if (a->mode == NM_ACT_MASKED) {
        g.prologue = a->x_meta != nullptr ? nml::PRO_MASK : nml::PRO_NONE;
        g.x_mask = (const uint32_t*)a->x_meta;
        if (a->x_meta == nullptr && use_few(T, R)) return run_dense_few(g, part, part_avail, s);
        return run_dense_large(g, part, part_avail, s);
      }

      // ACT_DYNAMIC with the activation mitigations: the shifted selection (and the VAR
      // factor) into the workspace, then the product with the epilogue terms
      if (a->pts != 0) {
        if (!have_ws) return NM_EINVAL;
        const bool dyn = (a->pts & NM_PTS_DYNAMIC) != 0, var = (a->pts & NM_PTS_VAR) != 0;
        uint16_t* sx = (uint16_t*)a->workspace;
        float* mu = reinterpret_cast<float*>(reinterpret_cast<char*>(a->workspace) + align256(T * K * 2));
        float* alpha = mu + align256(T * 4) / 4;
        hipError_t e = nml::launch_select_pts(a->m, (const uint16_t*)a->x, T, K, a->ldx, a->n, dyn ? 1 : 0,
                                              (a->pts & NM_PTS_STATIC) ? a->pts_shift : nullptr, var ? 1 : 0, sx, K,
                                              a->x_mask_out, dyn ? mu : nullptr, var ? alpha : nullptr, s);
        if (e != hipSuccess) return NM_EHIP;
        R.note(NM_TAKEN_SELECT);
        g.x = sx; g.ldx = K; g.prologue = nml::PRO_NONE;
        g.row_scale = var ? alpha : nullptr;
        g.row_shift = dyn ? mu : nullptr;
        g.col_shift = a->col_shift;
        if (use_few(T, R)) return run_dense_few(g, part, part_avail, s);
        return run_dense_large(g, part, part_avail, s);
      }
      // ACT_DYNAMIC, one token with K-major weights: select and gather the kept K-rows
      if (gather1_route(a)) {
        const int64_t need = nml::gather1_part_bytes(K, O, a->m);
        if (a->workspace != nullptr && a->workspace_bytes >= need)
          return hip_status(nml::launch_gather1(a->m, (const uint16_t*)a->x, K, a->n, (const uint16_t*)a->w_kmajor, O,
                                                a->y, a->accumulate, a->x_mask_out, (float*)a->workspace,
                                                a->workspace_bytes, R, s));
      }
      // ACT_DYNAMIC, one token, no mask asked for, n = m/2: the weight-streaming kernel
      // selects inside the X row it stages, with no separate select pass
      if (T == 1 && have_ws && a->x_mask_out == nullptr && 2 * a->n == a->m) {
        nml::GemmArgs g1 = g;
        g1.x = (const uint16_t*)a->x; g1.ldx = a->ldx; g1.prologue = nml::PRO_NONE;
        if (!few_use_tile(g1)) {
          nml::FewArgs f = few_dense_args(g1);
          f.sel_m = a->m;
          if (nml::few_select_in_kernel(f)) return hip_status(nml::launch_few(f, part, part_avail, s));
        }
      }
      // ACT_DYNAMIC, few tokens: select into S(X), then stream the weights.  For 2-32
      // tokens on the streaming kernel S(X) is staged in 16-token blocks, so that each X
      // fragment load of the kernel reads 8 whole cache lines instead of 16 half lines.
      if (use_few(T, R) && have_ws) {
        uint16_t* sx = (uint16_t*)a->workspace;
        g.x = sx; g.ldx = K; g.prologue = nml::PRO_NONE;
        const bool blk = T >= 2 && T <= 32 && K % 32 == 0 && (a->m == 4 || a->m == 8 || a->m == 16 || a->m == 32) &&
                         !R.has(NM_ROUTE_ROW_SX) && !few_use_tile(g);
        hipError_t e = nml::launch_select(a->m, (const uint16_t*)a->x, T, K, a->ldx, a->n, sx, K, a->x_mask_out,
                                          nullptr, nullptr, 0, s, blk ? 1 : 0);
        if (e != hipSuccess) return NM_EHIP;
        R.note(NM_TAKEN_SELECT);
        if (blk) {
          nml::FewArgs f = few_dense_args(g);
          f.seg[0].loader = nml::XL_BLK;
          f.seg[0].ldx = K * 16;
          return hip_status(nml::launch_few(f, part, part_avail, s));
        }
        return run_dense_few(g, part, part_avail, s);
      }

      // ACT_DYNAMIC 2:4 under the NM_ROUTE_ACT_SPARSE_X hint: compress X once, then the
      // sparse matrix instruction with X as the sparse operand (register-staged tiles,
      // transposed output).  Measured on gfx950 slower than S(X) on the direct-to-LDS
      // dense tiles at every size: 4096 x 14336 at 256 / 8192 tokens 392 / 1315 us against
      // 62 / 805 us, 14336 x 4096 at 1024 tokens 302 against 124 us.
      if (R.has(NM_ROUTE_ACT_SPARSE_X) && a->n == 2 && a->m == 4 && !fp8 && a->w_scale == nullptr && have_ws) {
        uint16_t* xv = (uint16_t*)a->workspace;
        uint8_t* xm = (uint8_t*)a->workspace + ((T * (K / 2) * 2 + 15) / 16) * 16;
        hipError_t e = nml::launch_select(4, (const uint16_t*)a->x, T, K, a->ldx, 2, nullptr, 0, a->x_mask_out,
                                          xv, xm, 1, s);
        if (e != hipSuccess) return NM_EHIP;
        R.note(NM_TAKEN_SELECT);
        nml::SparseArgs sa{};
        sa.route = R;
        sa.w_vals = xv; sa.w_meta = xm; sa.kc = K;
        sa.x = (const uint16_t*)a->w; sa.ldx = a->ldw; sa.loader = nml::XL_PLAIN;
        sa.t = O; sa.o = T; sa.y = a->y; sa.ldy = a->ldy; sa.accumulate = a->accumulate; sa.trans_out = 1;
        return hip_status(nml::launch_gemm_sparse(sa, s));
      }
      const ActRoute route = act_route(R);
      uint32_t* mask = a->x_mask_out;
      if (route == ROUTE_SX && have_ws) {
        uint16_t* sx = (uint16_t*)a->workspace;
        hipError_t e = nml::launch_select(a->m, (const uint16_t*)a->x, T, K, a->ldx, a->n, sx, K, mask,
                                          nullptr, nullptr, 0, s);
        if (e != hipSuccess) return NM_EHIP;
        R.note(NM_TAKEN_SELECT);
        g.prologue = nml::PRO_NONE; g.x = sx; g.ldx = K;
        const int64_t widen = fp8_widen_bytes(a), woff = align256(stage);
        int64_t poff = woff;   // [S(X)][widened W][partial sums]
        if (widen > 0 && a->workspace_bytes >= woff + widen) {
          uint16_t* wb = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(a->workspace) + woff);
          e = nml::launch_widen_fp8((const uint8_t*)a->w, a->ldw, O, K, wb, s);
          if (e != hipSuccess) return NM_EHIP;
          R.note(NM_TAKEN_WIDEN);
          g.w = wb; g.ldw = K; g.w_fp8 = 0;   // w_scale stays: applied in the epilogue
          poff = woff + align256(widen);
        }
        int64_t pavail = 0;
        float* pp = ws_slice(a->workspace, a->workspace_bytes, poff, &pavail);
        return run_dense_large(g, pp, pavail, s);
      }
      if (route == ROUTE_MASK && (mask != nullptr || have_ws)) {
        if (mask == nullptr) mask = (uint32_t*)a->workspace;
        hipError_t e = nml::launch_select(a->m, (const uint16_t*)a->x, T, K, a->ldx, a->n, nullptr, 0, mask,
                                          nullptr, nullptr, 0, s);
        if (e != hipSuccess) return NM_EHIP;
        R.note(NM_TAKEN_SELECT);
        g.prologue = nml::PRO_MASK; g.x_mask = mask;
        return hip_status(nml::launch_gemm_dense(g, s));
      }
      g.prologue = nml::PRO_SELECT; g.mask_out = a->x_mask_out;
      return hip_status(nml::launch_gemm_dense(g, s));
    }
    case NM_W_COMPRESSED:
    case NM_W_SLIDE: {
      int64_t kc = K;
      int ns = 2;
      if (a->mode == NM_W_SLIDE) {
        ns = a->ns;
        if (ns < 2 || ns > 8) return ns > 8 ? NM_EUNSUPPORTED : NM_EINVAL;
        if (K % (2 * ns)) return NM_ESHAPE;
        kc = (K / (2 * ns)) * 4 * (ns - 1);
      } else if (K % 4) {
        return NM_ESHAPE;
      }
      if (a->w_meta_fmt != NM_META_2BIT) return NM_EUNSUPPORTED;
      if (a->w_dtype != NM_W_BF16 && a->w_dtype != NM_W_FP8E4M3) return NM_EINVAL;
      if ((st = check_bf16(a->x, T, K, a->ldx, true))) return st;
      if (O > 0 && kc > 0 && (a->w == nullptr || a->w_meta == nullptr)) return NM_EINVAL;
      if ((a->w && !aligned16(a->w)) || (a->w_meta && !aligned16(a->w_meta))) return NM_EALIGN;
      if (a->workspace != nullptr && !aligned16(a->workspace)) return NM_EALIGN;
      if (!span_ok(O, kc)) return NM_ESHAPE;
      if (a->w_dtype == NM_W_FP8E4M3) {
        // fp8 weights: the activations are quantized per token to e4m3 and lifted in one
        // pass, and the product runs on the fp8 sparse matrix instruction
        if (a->w_scale == nullptr && O > 0) return NM_EINVAL;
        if (a->w_scale != nullptr && !aligned16(a->w_scale)) return NM_EALIGN;
        if (kc % 128 != 0) return NM_EUNSUPPORTED;
        if ((st = bind_scratch())) return st;
        if (T == 0 || O == 0) return NM_OK;
        if (K == 0) return a->accumulate ? NM_OK : zero_output(a->y, T, O, a->ldy, s);
        return w8a8_product(a, kc, ns, s);
      }
      if ((st = bind_scratch())) return st;
      if (T == 0 || O == 0) return NM_OK;
      if (K == 0) return a->accumulate ? NM_OK : zero_output(a->y, T, O, a->ldy, s);
      const nml::Route R = route_of(a, true);
      if (use_few(T, R) || T > kFewMaxT) {
        // the split tile kernel (few tokens, or too few large tiles to fill the chip)
        const int64_t tile = w_mode_tile_bytes(a, kc, ns);
        if (tile == 0 || (tile > 0 && a->workspace != nullptr && a->workspace_bytes >= tile)) {
          nml::SparseArgs sa = w_mode_sparse_args(a, kc, ns, true);
          int64_t off = 0;
          if (a->mode == NM_W_SLIDE && !sa.lift_dma) {
            uint16_t* xl = (uint16_t*)a->workspace;
            hipError_t e = nml::launch_lift(ns, (const uint16_t*)a->x, T, K, a->ldx, xl, lift_ld(kc), s);
            if (e != hipSuccess) return NM_EHIP;
            R.note(NM_TAKEN_LIFT);
            sa.x = xl;
            off = align256(T * lift_ld(kc) * 2);
          }
          return hip_status(nml::launch_gemm_lds_sp_small(
              sa, reinterpret_cast<float*>(reinterpret_cast<char*>(a->workspace) + off), a->workspace_bytes - off, s));
        }
        if (use_few(T, R))
          return hip_status(nml::launch_few(few_sparse_args(a, kc, ns), (float*)a->workspace,
                                            a->workspace ? a->workspace_bytes : 0, s));
      }
      nml::SparseArgs sa{};
      sa.route = R;
      sa.w_vals = (const uint16_t*)a->w; sa.w_meta = (const uint8_t*)a->w_meta; sa.kc = kc;
      sa.x = (const uint16_t*)a->x; sa.ldx = a->ldx; sa.ns = ns;
      sa.loader = a->mode == NM_W_SLIDE ? nml::XL_LIFT : nml::XL_PLAIN;
      sa.t = T; sa.o = O; sa.y = a->y; sa.ldy = a->ldy; sa.accumulate = a->accumulate; sa.trans_out = 0;
      sa.lift_dma = w_lift_dma(a) ? 1 : 0;
      if (sa.lift_dma && !sparse_lds_large(sa)) sa.lift_dma = 0;   // register kernel: lift in its loader
      int64_t off = 0;
      if (a->mode == NM_W_SLIDE && !sa.lift_dma && a->workspace != nullptr && a->workspace_bytes >= T * lift_ld(kc) * 2) {
        // materialise lift(X) once so the product kernel reads X with 16-byte loads
        uint16_t* xl = (uint16_t*)a->workspace;
        hipError_t e = nml::launch_lift(ns, (const uint16_t*)a->x, T, K, a->ldx, xl, lift_ld(kc), s);
        if (e != hipSuccess) return NM_EHIP;
        R.note(NM_TAKEN_LIFT);
        sa.x = xl; sa.ldx = lift_ld(kc); sa.loader = nml::XL_PLAIN;
        off = align256(T * lift_ld(kc) * 2);
      }
      if ((st = use_meta_block(sa, a->workspace, a->workspace_bytes, off, s))) return st;
      if (const int64_t sp = sparse_splits(sa); sp > 1) {
        // [lifted X][K-blocked positions][partial sums]
        const int64_t poff = off + (sa.w_meta_blk != nullptr ? align256(nml::meta_block_bytes(sa.o, sa.kc)) : 0);
        int64_t avail = 0;
        float* part = ws_slice(a->workspace, a->workspace_bytes, poff, &avail);
        return hip_status(nml::launch_gemm_lds_sp_split(sa, sp, part, avail, s));
      }
      return hip_status(nml::launch_gemm_sparse(sa, s));
    }
    default:
      return NM_EINVAL;
  }
}

}  // namespace

extern "C" {

nm_status nm_spmm(const nm_spmm_args* a, void* stream) { return spmm_impl(a, stream, false); }

nm_status nm_spmm_noalloc(const nm_spmm_args* a, void* stream) { return spmm_impl(a, stream, true); }


// ------------------------------------------------------------- Spense GLU layout ---

int64_t nm_spense_glu_order_workspace_size(int64_t inter) {
  return inter <= 0 ? 0 : align256(inter * 8) + inter * 4;
}

nm_status nm_spense_glu_order(const void* w_gate, const void* w_up, int64_t ld_gu, const void* w_down, int64_t ld_d,
                              int64_t hidden, int64_t inter, const double* hs_in, const double* hs_mid,
                              int64_t n_dense, nm_spense_strategy strategy, int32_t* perm, double* scores,
                              void* workspace, int64_t workspace_bytes, void* stream) {
  if (hidden < 0 || inter < 0 || inter > 0x7FFFFFFF || n_dense < 0 || n_dense > inter) return NM_ESHAPE;
  if (strategy != NM_SPENSE_LOSS && strategy != NM_SPENSE_TAIL) return NM_EINVAL;
  if (inter > 0 && (perm == nullptr || workspace == nullptr ||
                    workspace_bytes < nm_spense_glu_order_workspace_size(inter)))
    return NM_EINVAL;
  nm_status st;
  if (strategy == NM_SPENSE_LOSS) {
    if ((st = check_bf16(w_gate, inter, hidden, ld_gu, true))) return st;
    if ((st = check_bf16(w_up, inter, hidden, ld_gu, true))) return st;
    if ((st = check_bf16(w_down, hidden, inter, ld_d, true))) return st;
    if ((hs_in == nullptr && hidden > 0) || (hs_mid == nullptr && inter > 0)) return NM_EINVAL;
    if ((hs_in && !aligned16(hs_in)) || (hs_mid && !aligned16(hs_mid))) return NM_EALIGN;
  }
  if ((perm && !aligned16(perm)) || (scores && !aligned16(scores)) || (workspace && !aligned16(workspace)))
    return NM_EALIGN;
  if (inter == 0) return NM_OK;
  const hipStream_t s = as_stream(stream);
  double* sc = scores != nullptr ? scores : reinterpret_cast<double*>(workspace);
  int32_t* flag = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(workspace) + align256(inter * 8));
  hipError_t e;
  if (strategy == NM_SPENSE_LOSS) {
    e = nml::launch_glu_scores((const uint16_t*)w_gate, (const uint16_t*)w_up, ld_gu, (const uint16_t*)w_down, ld_d,
                               hidden, inter, hs_in, hs_mid, sc, s);
    if (e == hipSuccess) e = nml::launch_rank_flags(sc, inter, n_dense, flag, s);
  } else {
    e = nml::launch_tail_flags(inter, n_dense, flag, s);
  }
  if (e == hipSuccess) e = nml::launch_flag_lists(flag, inter, n_dense, perm, perm + (inter - n_dense), s);
  return hip_status(e);
}

int64_t nm_spense_pack_workspace_size(int64_t o, int64_t k, int axis, int64_t n_sparse) {
  if (axis != 0 || o <= 0 || k <= 0 || n_sparse <= 0) return 0;
  return n_sparse * ((k + 7) / 8 * 8) * 2;   // the gathered sparse rows
}

nm_status nm_spense_pack(const void* w, int64_t o, int64_t k, int64_t ldw, int axis, const int32_t* perm,
                         int64_t n_sparse, void* ws_values, void* ws_meta, nm_meta fmt, void* wd, int64_t ldwd,
                         void* workspace, int64_t workspace_bytes, void* stream) {
  if (axis != 0 && axis != 1) return NM_EINVAL;
  if (fmt != NM_META_U8 && fmt != NM_META_2BIT) return NM_EINVAL;
  if (o < 0 || k < 0) return NM_ESHAPE;
  const int64_t n = axis == 0 ? o : k;
  if (n_sparse < 0 || n_sparse > n || n > 0x7FFFFFFF) return NM_ESHAPE;
  const int64_t kc = axis == 0 ? k : n_sparse;                  // reduction length of the 2:4 region
  const int64_t srows = axis == 0 ? n_sparse : o;               // rows of the 2:4 region
  const int64_t drows = axis == 0 ? o - n_sparse : o, dcols = axis == 0 ? k : k - n_sparse;
  if (srows > 0 && kc > 0 && (kc % 4) != 0) return NM_ESHAPE;
  nm_status st;
  if ((st = check_bf16(w, o, k, ldw, true))) return st;
  if (n > 0 && perm == nullptr) return NM_EINVAL;
  if (srows > 0 && kc > 0 && (ws_values == nullptr || ws_meta == nullptr)) return NM_EINVAL;
  if ((st = check_bf16(wd, drows, dcols, ldwd, true))) return st;
  if ((perm && !aligned16(perm)) || (ws_values && !aligned16(ws_values)) || (ws_meta && !aligned16(ws_meta)) ||
      (workspace && !aligned16(workspace)))
    return NM_EALIGN;
  const int64_t need = nm_spense_pack_workspace_size(o, k, axis, n_sparse);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return NM_EINVAL;
  if (o == 0 || k == 0) return NM_OK;
  const hipStream_t s = as_stream(stream);
  const int m2 = fmt == NM_META_2BIT ? 1 : 0;
  hipError_t e = hipSuccess;
  if (axis == 0) {
    // output-split: gather the sparse rows, compress them 2:4 along K; gather the dense rows
    if (n_sparse > 0) {
      uint16_t* g = reinterpret_cast<uint16_t*>(workspace);
      const int64_t ldg = (k + 7) / 8 * 8;
      e = nml::launch_gather_rows((const uint16_t*)w, ldw, o, k, perm, n_sparse, g, ldg, s);
      if (e == hipSuccess)
        e = nml::launch_select(4, g, n_sparse, k, ldg, 2, nullptr, 0, nullptr, (uint16_t*)ws_values,
                               (uint8_t*)ws_meta, m2, s);
    }
    if (e == hipSuccess && drows > 0)
      e = nml::launch_gather_rows((const uint16_t*)w, ldw, o, k, perm + n_sparse, drows, (uint16_t*)wd, ldwd, s);
  } else {
    // input-split: 2:4 over the columns perm[0:n_sparse], dense columns perm[n_sparse:k]
    e = nml::launch_pack_cols((const uint16_t*)w, o, ldw, k, perm, n_sparse, (uint16_t*)ws_values,
                              (uint8_t*)ws_meta, m2, s);
    if (e == hipSuccess)
      e = nml::launch_gather_cols((const uint16_t*)w, o, ldw, k, perm + n_sparse, dcols, (uint16_t*)wd, ldwd, s);
  }
  return hip_status(e);
}

// the two parts of an output-split call as nm_spmm calls
static nm_spmm_args outsplit_part(int sparse, const void* x, int64_t t, int64_t k, int64_t ldx, const void* w,
                                  const void* meta, int64_t o, int64_t ldw, float* y, int64_t ldy, int accumulate) {
  nm_spmm_args a{};
  a.mode = sparse ? NM_W_COMPRESSED : NM_ACT_MASKED;
  a.n = sparse ? 2 : 4; a.m = 4; a.ns = 2;
  a.t = t; a.o = o; a.k = k;
  a.x = x; a.ldx = ldx;
  a.w = w; a.ldw = ldw; a.w_dtype = NM_W_BF16;
  a.w_meta = meta; a.w_meta_fmt = NM_META_2BIT;
  a.y = y; a.ldy = ldy; a.accumulate = accumulate;
  return a;
}

int64_t nm_spense_outsplit_workspace_size(int64_t t, int64_t k, int64_t o_s, int64_t o_d) {
  if (t <= 0 || k <= 0 || o_s < 0 || o_d < 0) return 0;
  int64_t nb = 0;
  if (o_s > 0) {
    const nm_spmm_args a = outsplit_part(1, nullptr, t, k, k, nullptr, nullptr, o_s, k / 2, nullptr, o_s + o_d, 0);
    nb = nm_spmm_workspace_size(&a);
  }
  if (o_d > 0) {
    const nm_spmm_args b = outsplit_part(0, nullptr, t, k, k, nullptr, nullptr, o_d, k, nullptr, o_s + o_d, 0);
    const int64_t nd = nm_spmm_workspace_size(&b);
    nb = nd > nb ? nd : nb;
  }
  return nb;
}

nm_status nm_spense_outsplit_gemm(const void* x, int64_t t, int64_t k, int64_t ldx, const void* ws_values,
                                  const void* ws_meta, int64_t o_s, const void* wd, int64_t ldwd, int64_t o_d,
                                  float* y, int64_t ldy, int accumulate, void* workspace, int64_t workspace_bytes,
                                  void* stream) {
  if (t < 0 || k < 0 || o_s < 0 || o_d < 0) return NM_ESHAPE;
  if (k % 4) return NM_ESHAPE;
  if (ldy < o_s + o_d) return NM_ESHAPE;
  if (o_s > 0 && o_d > 0 && (o_s % 4) != 0) return NM_EALIGN;   // the dense part starts at y + o_s
  nm_status st = NM_OK;
  if (o_s > 0) {
    nm_spmm_args a = outsplit_part(1, x, t, k, ldx, ws_values, ws_meta, o_s, k / 2, y, ldy, accumulate);
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    if ((st = nm_spmm(&a, stream))) return st;
  }
  if (o_d > 0) {
    nm_spmm_args b = outsplit_part(0, x, t, k, ldx, wd, nullptr, o_d, ldwd, y != nullptr ? y + o_s : nullptr, ldy,
                                   accumulate);
    b.workspace = workspace; b.workspace_bytes = workspace_bytes;
    st = nm_spmm(&b, stream);
  }
  return st;
}

int64_t nm_hybrid_pack_workspace_size(int64_t k) { return k <= 0 ? 0 : k * 12 + 64; }

nm_status nm_hybrid_pack(const void* w, int64_t o, int64_t k, int64_t ldw, int64_t k_dense, int32_t* sparse_cols,
                         int32_t* dense_cols, void* ws_values, void* ws_meta, nm_meta fmt, void* wd, int64_t ldwd,
                         void* workspace, int64_t workspace_bytes, void* stream) {
  if (o < 0 || k < 0 || k_dense < 0 || k_dense > k || k > 65536) return NM_ESHAPE;
  if (((k - k_dense) % 4) != 0) return NM_ESHAPE;
  if (fmt != NM_META_U8 && fmt != NM_META_2BIT) return NM_EINVAL;
  nm_status st;
  if ((st = check_bf16(w, o, k, ldw, true))) return st;
  const int64_t ks = k - k_dense;
  if (k > 0 && workspace_bytes < nm_hybrid_pack_workspace_size(k)) return NM_EINVAL;
  if (k > 0 && workspace == nullptr) return NM_EINVAL;
  if (ks > 0 && (sparse_cols == nullptr || (o > 0 && (ws_values == nullptr || ws_meta == nullptr)))) return NM_EINVAL;
  if (k_dense > 0 && dense_cols == nullptr) return NM_EINVAL;
  if (k_dense > 0 && (st = check_bf16(wd, o, k_dense, ldwd, true))) return st;
  if ((sparse_cols && !aligned16(sparse_cols)) || (dense_cols && !aligned16(dense_cols)) ||
      (ws_values && !aligned16(ws_values)) || (ws_meta && !aligned16(ws_meta)) ||
      (workspace && !aligned16(workspace)))
    return NM_EALIGN;
  if (k == 0) return NM_OK;
  return hip_status(nml::launch_hybrid_pack((const uint16_t*)w, o, k, ldw, k_dense, sparse_cols, dense_cols,
                                            (uint16_t*)ws_values, (uint8_t*)ws_meta, fmt == NM_META_2BIT ? 1 : 0,
                                            (uint16_t*)wd, ldwd, workspace, as_stream(stream)));
}

int64_t nm_hybrid_gemm_workspace_size(int64_t t, int64_t k_s, int64_t k_d, int64_t o, int gathered, uint32_t route) {
  if (t <= 0 || o <= 0 || k_s < 0 || k_d < 0 || (k_s == 0 && k_d == 0)) return 0;
  nml::Route r{};
  r.flags = route;
  const int64_t stage = gathered ? t * hybrid_ldp(k_s, k_d) * 2 : 0;
  int64_t part = 0;
  if (use_few(t, r) || t > kFewMaxT) {
    const int64_t ldp = gathered ? hybrid_ldp(k_s, k_d) : k_s + k_d;
    const nml::SparseArgs sa = hybrid_sparse_args(nullptr, ldp, gathered ? hybrid_off1(k_s) : k_s, t, k_s, k_d,
                                                  nullptr, nullptr, nullptr, k_d, o, nullptr, o, 0, r);
    if (sp_few_tile(sa)) part = nml::gemm_lds_sp_small_part_bytes(sa);
    else if (use_few(t, r))
      part = nml::few_partial_bytes(few_hybrid_args(nullptr, ldp, 0, t, k_s, k_d, nullptr, nullptr, nullptr, k_d, o,
                                                    nullptr, o, 0, r));
  }
  if (part > 0) return align256(stage) + part;
  if (!use_few(t, r)) {
    // large-token product: [permuted X][K-blocked positions][partial sums of split tiles]
    const int64_t ldp = gathered ? hybrid_ldp(k_s, k_d) : k_s + k_d;
    const nml::SparseArgs sa = hybrid_sparse_args(nullptr, ldp, gathered ? hybrid_off1(k_s) : k_s, t, k_s, k_d,
                                                  nullptr, nullptr, nullptr, k_d, o, nullptr, o, 0, r);
    const int64_t mb = k_s > 0 ? meta_block_ws(sa) : 0, sp = sparse_splits(sa);
    if (mb > 0 || sp > 1) return align256(stage) + align256(mb) + (sp > 1 ? sp * t * o * 4 : 0);
  }
  return stage;
}

nm_status nm_hybrid_gemm(const void* x, int64_t t, int64_t ldx, const int32_t* sparse_cols, int64_t k_s,
                         const int32_t* dense_cols, int64_t k_d, const void* ws_values, const void* ws_meta,
                         nm_meta fmt, const void* wd, int64_t ldwd, int64_t o, float* y, int64_t ldy,
                         int accumulate, void* workspace, int64_t workspace_bytes, uint32_t route,
                         uint32_t* route_taken, void* stream) {
  if (t < 0 || o < 0 || k_s < 0 || k_d < 0) return NM_ESHAPE;
  if ((k_s % 4) != 0) return NM_ESHAPE;
  if (accumulate != 0 && accumulate != 1) return NM_EINVAL;
  if (fmt != NM_META_2BIT) return (fmt == NM_META_U8) ? NM_EUNSUPPORTED : NM_EINVAL;
  const bool gathered = sparse_cols != nullptr || dense_cols != nullptr;
  if (gathered && ((k_s > 0 && sparse_cols == nullptr) || (k_d > 0 && dense_cols == nullptr))) return NM_EINVAL;
  const int64_t kx = k_s + k_d;      // columns of x (the column lists index into them)
  nm_status st;
  if (x == nullptr && t > 0) return NM_EINVAL;
  if (x != nullptr) {
    if (ldx < kx || !span_ok(t, ldx)) return NM_ESHAPE;
    if (!aligned16(x) || (ldx % 8) != 0) return NM_EALIGN;
  }
  if (!gathered && (k_s % 8) != 0 && k_d > 0) return NM_EALIGN;
  if (o > 0 && k_s > 0 && (ws_values == nullptr || ws_meta == nullptr)) return NM_EINVAL;
  if ((ws_values && !aligned16(ws_values)) || (ws_meta && !aligned16(ws_meta))) return NM_EALIGN;
  if (k_d > 0 && (st = check_bf16(wd, o, k_d, ldwd, true))) return st;
  if (t > 0 && o > 0 && y == nullptr) return NM_EINVAL;
  if (y != nullptr) {
    if (ldy < o || !span_ok(t, ldy)) return NM_ESHAPE;
    if (!aligned16(y)) return NM_EALIGN;
  }
  if ((sparse_cols && !aligned16(sparse_cols)) || (dense_cols && !aligned16(dense_cols))) return NM_EALIGN;
  if (workspace != nullptr && !aligned16(workspace)) return NM_EALIGN;
  if (workspace_bytes < 0) return NM_EINVAL;
  // the gathered form stages the column-permuted X in the workspace
  const int64_t stage = gathered ? t * hybrid_ldp(k_s, k_d) * 2 : 0;
  if (gathered && t > 0 && o > 0 && (workspace == nullptr || workspace_bytes < stage)) return NM_EINVAL;
  if (t == 0 || o == 0) return NM_OK;
  const hipStream_t s = as_stream(stream);
  if (k_s == 0 && k_d == 0) return accumulate ? NM_OK : zero_output(y, t, o, ldy, s);

  nml::Route R{};
  R.flags = route;
  R.taken = route_taken;
  const uint16_t* xa = (const uint16_t*)x;
  int64_t lda = ldx, dbase = k_s;
  if (gathered) {
    uint16_t* xp = (uint16_t*)workspace;
    const int64_t ldp = hybrid_ldp(k_s, k_d);
    hipError_t e = nml::launch_permute_cols((const uint16_t*)x, t, ldx, kx, sparse_cols, k_s, dense_cols, k_d,
                                            hybrid_off1(k_s), xp, ldp, s);
    if (e != hipSuccess) return NM_EHIP;
    R.note(NM_TAKEN_PERMUTE);
    xa = xp; lda = ldp; dbase = hybrid_off1(k_s);
  }
  nml::SparseArgs sa = hybrid_sparse_args(xa, lda, dbase, t, k_s, k_d, ws_values, ws_meta, wd, ldwd, o, y, ldy,
                                          accumulate, R);
  if (use_few(t, R) || t > kFewMaxT) {
    // the split tile kernel (few tokens, or too few large tiles to fill the chip)
    int64_t avail = 0;
    float* part = ws_slice(workspace, workspace_bytes, stage > 0 ? align256(stage) : 0, &avail);
    if (sp_few_tile(sa) && avail >= nml::gemm_lds_sp_small_part_bytes(sa))
      return hip_status(nml::launch_gemm_lds_sp_small(sa, part, avail, s));
    if (use_few(t, R))
      return hip_status(nml::launch_few(few_hybrid_args(xa, lda, dbase, t, k_s, k_d, ws_values, ws_meta, wd, ldwd, o,
                                                        y, ldy, accumulate, R),
                                        part, avail, s));
  }
  const int64_t soff = stage > 0 ? align256(stage) : 0;
  if ((st = use_meta_block(sa, workspace, workspace_bytes, soff, s))) return st;
  if (const int64_t sp = sparse_splits(sa); sp > 1) {
    // [permuted X][K-blocked positions][partial sums]
    const int64_t poff = soff + (sa.w_meta_blk != nullptr ? align256(nml::meta_block_bytes(sa.o, sa.kc)) : 0);
    int64_t avail = 0;
    float* part = ws_slice(workspace, workspace_bytes, poff, &avail);
    return hip_status(nml::launch_gemm_lds_sp_split(sa, sp, part, avail, s));
  }
  return hip_status(nml::launch_gemm_sparse(sa, s));
}

}  // extern "C"
