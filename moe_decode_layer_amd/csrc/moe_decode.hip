// Persistent MoE decode layer for MI355X (gfx950, CDNA4) behind the C ABI of
// include/moe_decode.h.
//
// One launch runs the whole layer.  Every workgroup stays resident and walks
// its own share of one global list of work items (the early items are
// static, item i belonging to workgroup i mod G; the tail is claimed from
// counters); an item that needs earlier results waits for a counter the
// producing items bump, then for the tags of its inputs.  Blocks that stay
// resident across stages, pass ready results on through tagged buffers and
// load weights while earlier stages still compute follow "FlyDSL Mono
// Kernels for High-Interactivity LLM Serving in ATOM" (sections "What FlyDSL
// Provides" and "MiniMax-M3: Connecting Attention and Experts"); the deadline
// on every wait follows "SGLang's Low-Latency Mode Boosts DeepSeek-V4.1-Flash
// Speed by 1.56x on AMD" (section "AMD keeps the layer resident").
//
// Item list, in this order (an item only waits on items earlier in the list;
// each workgroup takes its items in list order and all workgroups are
// resident together, so every wait is eventually satisfied -- and if they
// were not all resident, the deadline turns the stall into an error):
//   router          : logits of one expert for up to 8 rows (batches above
//                     16 rows: a 16-row x 16-expert MFMA tile, or part of
//                     its H, read from a tiled copy of the router rows)
//   top-k           : 4 rows, one per wave (only for batches above 16 rows;
//                     smaller batches select top-k in every workgroup)
//   shared gate/up  : 16 weight rows (8 gate + 8 up) of the shared expert
//   routed gate/up  : 16 weight rows of one routed expert      -- waits: routing
//   shared down     : 128 output rows of the shared expert     -- waits: its gate/up
//   routed down     : 128 output rows of one routed expert     -- waits: its gate/up
//   combine         : 4 (or 8) rows x 128 columns of y         -- waits: the down
//                                                                 items of those columns
// A gate/up or down item covers up to 64 rows of its expert (four 16-row
// MFMA blocks); experts with more rows get one item per 64 rows.  Batches
// above 16 rows at H = 4096, I = 512 use wide items instead: gate/up items of
// 64 weight rows and down items of 512 output rows, for up to 32 rows each,
// with the down and combine items ordered by column group (see
// gu_item_wide).  Results handed between workgroups carry the run's epoch
// (tagged words), so a producer never waits for its own stores: it bumps a
// counter and moves on.
//
// Pre-norm block runs (the NORM instantiations) add a prologue before the
// list: the input RMSNorm, one row per workgroup, each row handed on by a
// ready word (norm_rows, wait_rows); the combine then adds the residual.
// Clipped SwiGLU caps g and clamps u at a caller-set limit in every gate/up
// epilogue (+inf by default).
//
// Expert weights are re-laid out once, at create time, into tiles of 16
// weight rows x 64 K (1 KiB of FP8 or MXFP8, 512 B of MXFP4): lane l of a
// wave reads the l-th 16 (MXFP4: 8) bytes of a tile, so every wave-wide
// weight load is one contiguous block.  Lane l = (n, kq), n = l % 16,
// kq = l / 16, holds row n's K elements [8 kq, 8 kq + 8) of the tile's first
// 32-element group and the same of its second group: exactly the B operand
// of v_mfma_f32_16x16x32_bf16, one scale group per instruction.  The fp32
// result of each MFMA is multiplied by its group's scale (fp32, or E8M0 as
// a power of two) and accumulated.  FP8 e4m3fn and FP4 e2m1 -> bf16 are
// exact (v_cvt_scalef32_pk_bf16_fp8 / _fp4 with scale 1) and bf16 x bf16
// products are exact in fp32, so the only rounding before the declared bf16
// points is fp32 accumulation.  Activation rows are the A operand; rows past
// the expert's row count are zero.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <limits.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>

#include "moe_decode.h"

namespace {

// ----------------------------------------------------------------------------
// Fixed decomposition
// ----------------------------------------------------------------------------
constexpr int kWave = 64;
constexpr int kWaves = 4;                   // waves per workgroup
constexpr int kThreads = kWave * kWaves;
constexpr int kMBlock = 16;                 // rows per MFMA block
constexpr int kMRange = 64;                 // rows per expert item (<= 4 MFMA blocks)
constexpr int kRouterRows = 8;              // rows per router item (small batches)
constexpr int kRouterTile = 16;             // rows and experts per router tile (larger batches)
constexpr int kRouterKsMax = 8;             // a router tile's H may be split over up to 8 items
// Small batches: the logits are laid out [copy][E][lg_tp] (lg_tp = 8 or 16
// rows), so each expert's rows sit together and a 128-byte line has at most
// two writers (lines written piecewise by many workgroups become readable
// much later); every router item writes lg_copies copies and each workgroup
// reads one, so a line has a fraction of the workgroups as readers
constexpr int kLgCopies = 8;
constexpr int kDownRows = 128;              // output rows per down item (8 row blocks)
constexpr int kTileRows = 16;               // weight rows per tile
constexpr int kTileK = 64;                  // K elements per tile (two scale groups)
constexpr int kGroup = 32;
constexpr int kMaxTokens = 512;
constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 16;
constexpr size_t kXsMaxBytes = 64 * 1024;   // x kept in LDS up to this size
constexpr int kHsMaxI = 1024;               // h staged in LDS up to this intermediate width
constexpr int kFullTiles = 16;              // tiles per wave of the fully unrolled items (H 4096, I 512)
// Wide items (batches above 16 rows at H = 64 kWideTiles, I = 64 kWideQ2 .. 64 kWideQ2 + 128)
constexpr int kWideTiles = 16;              // K tiles per wave of a wide gate/up item
constexpr int kWideQ2 = 8;                  // K tiles of a down row block
constexpr int kWideRb = 4;                  // gate/up row blocks per wide item (one per wave at the end)
constexpr int kWideRows = 32;               // rows per wide expert item (two MFMA blocks)
constexpr int kWideDnBlocks = 8;            // down row blocks per wave (128 output rows)

constexpr int kCombineRows = 4;             // rows per combine item
// Counter block (int32 words).  Every counter sits on a 256-byte line of its
// own (kLine words apart): a line many workgroups poll or bump must not also
// carry another hot word.  There are two blocks: a run uses block
// (epoch & 1) and, at its start, clears the other one for the next run, so
// no run has to reset anything on its way out.
constexpr int kLine = 64;
constexpr int kCtrTopkDone = 1 * kLine;     // distributed top-k items done
constexpr int kClaimGroups = 8;             // claim counters (workgroup index mod 8)
constexpr int kCtrTicket = 4 * kLine;       // [kClaimGroups] next unclaimed dynamic item of each group
constexpr int kCtrHReady = (4 + kClaimGroups) * kLine;   // [E+S] gate/up publications per expert (E+S <= 257)
constexpr int kMaxRowGroups = 128;          // down column groups: H / 128 <= 128
constexpr int kCtrRgDone = kCtrHReady + 257 * kLine;   // [H/128] down-wave publications (<= 128)
// "go" flag raised once by the last distributed top-k item, polled by every
// workgroup: kGoLines copies, 1 KiB apart, so the pollers spread over memory
// channels
constexpr int kGoLines = 64;
constexpr int kGoStride = 256;              // words
constexpr int kCtrTopkGo = kCtrRgDone + kMaxRowGroups * kLine;
constexpr int kCtrHead = kCtrTopkGo + kGoLines * kGoStride;

// Arrival counters (64-bit, outside the counter blocks, never cleared).
// Workgroup b adds to counter b mod kArriveGroups; the workgroups of a group
// together add exactly kRunUnits per run (the group's first workgroup adds
// kRunUnits minus the rest of the group, every other one 1), so every value
// a run's fetch-add returns lies in [n kRunUnits, (n + 1) kRunUnits) for the
// run's index n, whatever order the workgroups arrive in.  The run's tag and
// counter block follow from n, so no per-run value travels in the kernel
// arguments and a captured graph can replay a launch as it stands.
constexpr int kArriveGroups = 8;
constexpr int kRunUnitsLog2 = 16;           // grids of up to 2^16 workgroups
constexpr unsigned long long kRunUnits = 1ull << kRunUnitsLog2;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define GLOBAL __attribute__((address_space(1)))
#define CONSTANT __attribute__((address_space(4)))
#define SHARED __attribute__((address_space(3)))

// Division of an index n < 2^23 by a fixed d > 0 as a multiply and a shift:
// with l = ceil(log2 d), s = 23 + l and m = ceil(2^s / d), n m / 2^s exceeds
// n / d by less than 1/d, so floor(n m / 2^s) = floor(n / d) (the round-up
// method of Granlund and Montgomery).  Per-word index arithmetic in the
// gathers would otherwise spend dozens of instructions on every division.
struct FDiv {
  uint32_t m, s, d;
};
static inline FDiv make_fdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  FDiv f;
  f.d = d;
  f.s = 23 + l;
  f.m = (uint32_t)(((1ull << f.s) + d - 1) / d);
  return f;
}
__device__ __forceinline__ uint32_t fdiv(uint32_t n, uint32_t m, uint32_t s) {
  return (uint32_t)(((uint64_t)n * m) >> s);
}

struct Params {
  int T, H, E, K, S, I;
  // inputs / outputs
  const uint16_t* x;
  uint16_t* y;
  const float* router_w;
  const float* router_b;   // [E] (without a bias: any readable [E] floats, unused)
  int has_bias;
  // expert weights in 16 x 64 tiles of the format (WFmt<fmt>::W per lane) and
  // one WFmt<fmt>::Scale per tile row
  const void* w13p;    // [E+S][2I/16][H/64][64] tiles
  const void* s13p;    // [E+S][2I/16][H/64][16]
  const void* w2p;     // [E+S][H/16][I/64][64]
  const void* s2p;     // [E+S][H/16][I/64][16]
  size_t w13_bytes, s13_bytes, w2_bytes, s2_bytes;   // packed sizes (page touching)
  // workspace.  Words handed between workgroups carry the run's epoch in
  // their high half (see "Tagged hand-offs" below).
  uint64_t* lgt;       // [T][E] router logits (fp32 bits | epoch); tiles: [router_ks][T][E] partials
  int* topk_idx;       // [T][K]  (distributed top-k only)
  float* topk_w;       // [T][K]
  uint64_t* h_scr;     // [T*K + T*S][I/2] two bf16 of h | epoch, rows grouped by expert
  uint64_t* o_scr;     // [T*K + T*S][H] expert outputs (fp32 bits | epoch)
  int* ctr_base;       // two counter blocks: a run uses block (run index & 1)
                       // and clears the other one for the next run
  int* status;         // in-kernel status word (0 = ok), outside the blocks
  unsigned long long* arrive;  // [kArriveGroups] arrival counters, kLine ints apart:
                               // each run adds exactly kRunUnits to every one
  // debug copies (nullable)
  int* dbg_idx;
  float* dbg_w;
  int* dbg_rank;
  int* dbg_count;
  float* dbg_logits;
  long long* trace;    // [trace_blocks][1 + trace_cap][4]
  int trace_blocks, trace_cap;
  // derived
  long long deadline_ticks;  // wall-clock ticks (100 MHz)
  int expire_waits;    // test control: every wait gives up at its first check
  int local_topk;      // 1: every workgroup selects top-k itself
  int lg_copies, lg_tp_log2;
  FDiv fd_x8;          // H / 8: 16-byte words of an x row
  FDiv fd_h2;          // I / 2: tagged words of an h row
  int n_rb13;          // gate/up row blocks per expert: I/8
  int n_q13;           // tiles along H: H/64
  int n_rb2;           // down row blocks: H/16
  int n_q2;            // tiles along I: I/64
  int n_rg;            // down row groups: ceil(H/128)
  int n_mr_sh;         // shared M-ranges: ceil(T/mrange) (0 without a shared expert)
  int nch;             // 64-row chunks: ceil(T/64)
  // item list boundaries
  int n_router, n_topk;
  int router_tiles;    // 1: router items are 16 x 16 MFMA tiles (batches above 16 rows)
  int router_ks;       // H split of a tile: item (tile, ks) writes partial logits ks
  int i_router_end, i_topk_end, i_pre_end;   // list: router, top-k, shared gate/up, then routed
  int n_sdn;           // shared down items
  int n_cmb;           // combine items: ceil(T / cmb_rows) * n_rg
  // LDS offsets (bytes)
  int lds_bm, lds_cp, lds_cnt, lds_base, lds_nmrb, lds_mrlist, lds_rows, lds_tki, lds_prow, lds_tkw,
      lds_red, lds_misc, lds_tks, lds_xs, lds_hs, lds_lg;
  int lds_bytes;
  int xs_stride;       // x rows in LDS (bf16 elements per row), 0 when x stays in global memory
  int hs_stride;       // h rows staged in LDS for a down item, 0 when read from global memory
  // (kept last: the fields above are the ones the small-batch path reads)
  int wide;            // 1: wide items (see gu_item_wide / dn_item_wide)
  int mrange;          // rows per expert item: 64, wide 32
  int n_gu_mr;         // gate/up items per M-range: n_rb13, wide n_rb13/4
  int n_dn_mr;         // down items per M-range: n_rg, wide H/512
  int h_rows_per_count;  // gate/up publications per row block come one per this many rows
  FDiv fd_k;           // K: the row of a (row, k) pair index
  int cmb_rows;        // rows per combine item: 8 for wide items with K <= 8 and T >= 128, else 4
  const f32x4* router_wt;  // [ceil(E/16)][H/16][64]: lane (n, kq) holds router row 16 et + n, K 16 s + 4 kq .. + 3
  // pre-norm block runs: x then points at xn, the normalised rows
  const uint16_t* x_in;    // [T][H] bf16 block input (the residual stream)
  const float* norm_w;     // [H] RMSNorm weight
  uint16_t* xn;            // [T][H] bf16 normalised rows (written by the kernel)
  int* norm_ready;         // [T] epoch of the run that last wrote each xn row
  uint16_t* dbg_norm;      // [T][H] copy of xn (nullable)
  float norm_eps;
  float swiglu_limit;      // clipped SwiGLU: g -> min(g, L), u -> clamp(u, -L, L); +inf: no clip
  int full;                // 1: the full-tile variant runs this call (host-side choice, see make_params)
  int gu_pair;             // 1: full-tile MXFP4 gate/up items cover two row blocks (n_gu_mr = n_rb13 / 2)
};
// The kernel reads its parameters in place, from the constant kernel-argument
// segment, so the compiler can reload a field with a scalar load instead of
// keeping every field resident in scalar registers.
typedef const CONSTANT Params KParams;

// ----------------------------------------------------------------------------
// Small device helpers
// ----------------------------------------------------------------------------
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16, round to nearest even (overflow to inf, NaN kept NaN): one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// 8 FP8 e4m3fn bytes (two dwords, little-endian) -> 8 bf16, exact.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 8 FP4 E2M1 codes (one dword; byte j holds codes 2j, 2j + 1 in its low and
// high nibble) -> 8 bf16, exact (v_cvt_scalef32_pk_bf16_fp4 with scale 1).
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t v) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 0);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 1);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 2);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 3);
  bf16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}

// E8M0 block scale 2^(e - 127) as fp32 (exact; e = 0 is the fp32 subnormal
// 2^-127, e = 255 NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  return __uint_as_float(e == 0u ? 0x00400000u : e == 255u ? 0x7fc00000u : e << 23);
}

// Expert weight formats (fixed at create).  Every format tiles a matrix into
// 16 rows x 64 K (two scale groups of 32); lane (n, kq) of a wave holds row
// n's K [32 g + 8 kq, 32 g + 8 kq + 8) of both groups g: the B operand of one
// v_mfma_f32_16x16x32_bf16 per group.  A wave-wide load of a tile is one
// contiguous block (1 KiB, MXFP4 512 B).
//   0 FP8: e4m3fn, one fp32 scale per group     (16 bytes per lane; scales f32x2 per row)
//   1 MXFP8: e4m3fn, one E8M0 scale per group   (16 bytes per lane; scales 2 bytes per row)
//   2 MXFP4: E2M1, one E8M0 scale per group     (8 bytes per lane; scales 2 bytes per row)
// Elements decode exactly to bf16; the group's scale multiplies the fp32
// result of its MFMA (a power of two for E8M0: exact).
constexpr int kFmtFp8 = 0, kFmtMxfp8 = 1, kFmtMxfp4 = 2;
template <int FMT> struct WFmt;
template <> struct WFmt<kFmtFp8> { typedef u32x4 W; typedef f32x2 Scale; };
template <> struct WFmt<kFmtMxfp8> { typedef u32x4 W; typedef uint16_t Scale; };
template <> struct WFmt<kFmtMxfp4> { typedef u32x2 W; typedef uint16_t Scale; };

template <int FMT>
__device__ __forceinline__ bf16x8 wdecode(const typename WFmt<FMT>::W& w, int g) {
  if constexpr (FMT == kFmtMxfp4) return fp4x8_to_bf16(w[g]);
  else return fp8x8_to_bf16(w[2 * g], w[2 * g + 1]);
}
// Scale of group g of an MX tile row.  (The FP8 format's fp32 scales are
// read at each use directly: routed through a helper, even an inlined one,
// they cost the items registers and spills.)
__device__ __forceinline__ float mx_scale(uint32_t s, int g) { return e8m0_to_f32((s >> (8 * g)) & 0xffu); }
// An MX group decoded with its E8M0 scale applied in the conversion: the
// scale is a power of two, so each scaled element is still exact in bf16
// (bf16 has fp32's exponent range) and the group's MFMA can accumulate
// straight into the item's sums.  The full-tile items use this form.
template <int FMT>
__device__ __forceinline__ bf16x8 wdecode_scaled(const typename WFmt<FMT>::W& w, int g, float sc) {
  static_assert(FMT != kFmtFp8, "FP8 scales are not powers of two");
  bf16x2 a, b, c, d;
  if constexpr (FMT == kFmtMxfp4) {
    a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[g], sc, 0);
    b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[g], sc, 1);
    c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[g], sc, 2);
    d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[g], sc, 3);
  } else {
    a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * g], sc, false);
    b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * g], sc, true);
    c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * g + 1], sc, false);
    d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * g + 1], sc, true);
  }
  bf16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}
__device__ __forceinline__ f32x4 mfma16_acc(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, zero, 0, 0, 0);
}

// Global-memory loads (explicit address space: no flat instructions).
template <typename T>
__device__ __forceinline__ T ld(const T* p) { return *(const GLOBAL T*)p; }
__device__ __forceinline__ u32x4 ld_stream(const u32x4* p) {
  return __builtin_nontemporal_load((const GLOBAL u32x4*)p);
}
// Group scales are also read once: streamed like the weights (cached loads
// of a once-read stream ran at less than half the bandwidth of streaming
// ones in a read-only sweep on this GPU).
__device__ __forceinline__ f32x2 ld_stream(const f32x2* p) {
  return __builtin_nontemporal_load((const GLOBAL f32x2*)p);
}
__device__ __forceinline__ uint16_t ld_stream(const uint16_t* p) {
  return __builtin_nontemporal_load((const GLOBAL uint16_t*)p);
}
__device__ __forceinline__ u32x2 ld_stream(const u32x2* p) {
  return __builtin_nontemporal_load((const GLOBAL u32x2*)p);
}
template <typename T>
__device__ __forceinline__ void st(T* p, T v) { *(GLOBAL T*)p = v; }

// DPP lane exchange within 16-lane rows (VALU, no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- 7 - i within 8
constexpr int kDppMirror = 0x140;     // lane i <- 15 - i within 16
constexpr int kDppRowShl1 = 0x101;    // lane i <- i + 1
constexpr int kDppRowRor8 = 0x128;    // lane i <- (i + 8) mod 16

// Sum over the 64 lanes, the same value in every lane, in a fixed order.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ int atomic_add_agent(int* p, int v) {
  return __hip_atomic_fetch_add((GLOBAL int*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int load_agent(int* p) {
  return __hip_atomic_load((GLOBAL int*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(int* p, int v) {
  __hip_atomic_store((GLOBAL int*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Data handed from one workgroup to another (logits, top-k, h, o) is written
// and read with device-scope relaxed atomic stores and loads: they go to the
// device coherence point instead of a workgroup's L1 or its XCD's L2, so no
// cache-wide write-back or invalidate is ever needed.  A producer waits until
// its stores are acknowledged (s_waitcnt) before it bumps a counter; a
// consumer reads the data only after it has seen the counter.
__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store((GLOBAL float*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(int* p, int v) {
  __hip_atomic_store((GLOBAL int*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(uint32_t* p, uint32_t v) {
  __hip_atomic_store((GLOBAL uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load((GLOBAL float*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_coh(const int* p) {
  return __hip_atomic_load((GLOBAL int*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u32x4 ld_coh16(const void* p) {
  const uint64_t a = __hip_atomic_load((GLOBAL uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t b = __hip_atomic_load((GLOBAL uint64_t*)p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return (u32x4){(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
}
// Wait until this wave's outstanding memory operations are acknowledged.
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0); }

// Timeline clock: read only when a trace buffer was given (a clock read
// costs a scalar-memory round trip).
__device__ __forceinline__ long long tl_clock(KParams& p) { return p.trace ? (long long)wall_clock64() : 0; }
__device__ __forceinline__ long long tl_cycles(KParams& p) {
  return p.trace ? (long long)__builtin_amdgcn_s_memtime() : 0;
}

// This workgroup's view of the run -- its tag (epoch) and counter block --
// is resolved at kernel entry from the arrival counters (see kArriveGroups)
// and carried in Lds (below) as uniform values.  Run n has epoch
// (n mod (2^32 - 1)) + 1 (never 0, the value of a cleared word) and uses
// counter block n & 1.
struct RunCtx {
  uint32_t epoch;
  uint32_t pad;
  int* ctr;
};
__shared__ RunCtx s_run;

// Tagged hand-offs.  Logits, h and expert outputs travel as 64-bit words:
// 32 bits of payload, and the run's epoch in the high half.  A 64-bit store
// is single-copy atomic, so a reader that sees the current epoch sees the
// payload written with it.  The producer therefore never waits for its
// stores before it counts itself done (the count only tells readers when to
// look); a reader that finds a stale tag reads the word again.
__device__ __forceinline__ void st_tag(uint64_t* p, uint32_t v, uint32_t epoch) {
  __hip_atomic_store((GLOBAL uint64_t*)p, (uint64_t)epoch << 32 | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_tag(const uint64_t* p) {
  return __hip_atomic_load((GLOBAL uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tag_ok(uint64_t v, uint32_t epoch) { return (uint32_t)(v >> 32) == epoch; }
// Counter bump whose result is not needed (no return trip is waited for).
__device__ __forceinline__ void count_done(int* p) {
  __hip_atomic_fetch_add((GLOBAL int*)p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// s_waitcnt vmcnt(n) (n <= 63), leaving the LDS and export counters alone:
// every vector memory operation of this wave except the n most recent is done.
template <int N>
__device__ __forceinline__ void wait_vm_older_than() {
  static_assert(N >= 0 && N <= 63, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// A down wave counts itself in for its column group only once its output
// stores have landed, so a combine that sees the count finds the outputs
// tagged on its first read.  To keep the wave from stalling on that, the
// count is deferred ("pending") to the next item, right after that item has
// issued its own loads (N of them): waiting then for everything older costs
// nothing.  Items that issue no loads first flush with a full wait.
template <int N>
__device__ __forceinline__ void flush_pending(int* ctr, int& pend) {
  if (pend >= 0) {
    wait_vm_older_than<N>();
    if (lane_id() == 0) count_done(ctr + kCtrRgDone + pend * kLine);
    pend = -1;
  }
}
// The same with N + extra operations younger than the stores, extra in
// [0, 8] known only at run time (uniform).
template <int N>
__device__ __forceinline__ void flush_pending_rt(int* ctr, int& pend, int extra) {
  static_assert(N + 8 <= 63, "vmcnt is 6 bits");
  if (pend >= 0) {
    switch (extra) {
      case 0: wait_vm_older_than<N>(); break;
      case 1: wait_vm_older_than<N + 1>(); break;
      case 2: wait_vm_older_than<N + 2>(); break;
      case 3: wait_vm_older_than<N + 3>(); break;
      case 4: wait_vm_older_than<N + 4>(); break;
      case 5: wait_vm_older_than<N + 5>(); break;
      case 6: wait_vm_older_than<N + 6>(); break;
      case 7: wait_vm_older_than<N + 7>(); break;
      default: wait_vm_older_than<N + 8>(); break;
    }
    if (lane_id() == 0) count_done(ctr + kCtrRgDone + pend * kLine);
    pend = -1;
  }
}
__device__ __forceinline__ void flush_pending_now(int* ctr, int& pend) {
  if (pend >= 0) {
    wait_stores();
    if (lane_id() == 0) count_done(ctr + kCtrRgDone + pend * kLine);
    pend = -1;
  }
}

// The copy of a go flag this workgroup polls.
__device__ __forceinline__ int* go_flag(int* base) { return base + (blockIdx.x % kGoLines) * kGoStride; }

// Thread 0 publishes "one more item done" on *ctr once every wave's stores of
// the item are acknowledged.  With a flag, the last of `target` items also
// raises the flag (one write that many waiters poll instead of the contended
// counter).
__device__ void publish_done(int* ctr, int target = 0, int* flag = nullptr) {
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = atomic_add_agent(ctr, 1);
    if (flag && old == target - 1)
      for (int i = 0; i < kGoLines; ++i) store_agent(flag + i * kGoStride, 1);
  }
}

// Workgroup-wide wait until *ctr >= target.  Thread 0 polls under a
// deadline; the pause between polls starts at ~0.05 us and, after max_fast
// short ones, doubles up to ~0.9 us, so long waits load the polled line
// lightly.  The result is broadcast through LDS, and the barrier orders
// every wave's later loads after it.  false: deadline passed or another
// workgroup reported an error.
__device__ bool wait_geq(KParams& p, int* ctr, int target, SHARED int* lds_flag, int max_fast = 8) {
  if (threadIdx.x == 0) {
    int ok = 1;
    if (load_agent(ctr) < target) {
      const long long t_end = (long long)wall_clock64() + (p.expire_waits ? 0 : p.deadline_ticks);
      int spins = 0;
      while (true) {
        if (load_agent(ctr) >= target) break;
        if ((spins & 7) == 7 && load_agent(p.status) != 0) { ok = 0; break; }
        if ((long long)wall_clock64() > t_end) {
          int expected = 0;
          __hip_atomic_compare_exchange_strong((GLOBAL int*)(p.status), &expected, MOE_ERR_TIMEOUT,
                                               __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
          ok = 0;
          break;
        }
        const int step = spins - max_fast;
        if (step < 0) __builtin_amdgcn_s_sleep(2);
        else if (step < 2) __builtin_amdgcn_s_sleep(4);
        else if (step < 4) __builtin_amdgcn_s_sleep(8);
        else if (step < 6) __builtin_amdgcn_s_sleep(16);
        else __builtin_amdgcn_s_sleep(32);
        ++spins;
      }
    }
    *lds_flag = ok;
    // when the last wait ended (read back by the same thread for the timeline)
    *(SHARED long long*)(lds_flag + 11) = tl_clock(p);
  }
  __syncthreads();
  const int ok = *lds_flag;
  __syncthreads();
  return ok != 0;
}

// Copy n 16-byte (or 8-byte) words with the whole workgroup, kBatch loads in
// flight per thread before any LDS write, so a copy costs about one memory
// round trip per kBatch * kThreads words instead of one per kThreads.
constexpr int kBatch = 8;
template <typename Word, typename LoadFn, typename StoreFn>
__device__ __forceinline__ void batched_copy(int n, LoadFn load, StoreFn store) {
  for (int i0 = threadIdx.x; i0 < n; i0 += kBatch * kThreads) {
    Word v[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int i = i0 + b * kThreads;
      if (i < n) v[b] = load(i);
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int i = i0 + b * kThreads;
      if (i < n) store(i, v[b]);
    }
  }
}

// Workgroup-wide OR of one predicate per thread (slots: kWaves LDS words).
__device__ __forceinline__ bool block_any(bool v, SHARED int* slots) {
  const unsigned long long b = __ballot(v);
  if (lane_id() == 0) slots[wave_id()] = b != 0ull;
  __syncthreads();
  int any = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) any |= slots[i];
  __syncthreads();
  return any != 0;
}

// Thread 0 checks the deadline (started at *t_end == 0) between polling
// rounds, and every 8th round (counted in *round) the error status, then
// pauses; the verdict is broadcast through LDS.  The status is read only now
// and then because its round trip would otherwise double every round's.
__device__ bool poll_round(KParams& p, long long* t_end, int* round, SHARED int* lds_flag) {
  if (threadIdx.x == 0) {
    int ok = 1;
    const long long now = (long long)wall_clock64();
    if (*t_end == 0) *t_end = now + (p.expire_waits ? 0 : p.deadline_ticks);
    if (now > *t_end) {
      int expected = 0;
      __hip_atomic_compare_exchange_strong((GLOBAL int*)(p.status), &expected, MOE_ERR_TIMEOUT,
                                           __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ok = 0;
    } else if ((++*round & 7) == 0 && load_agent(p.status) != 0) {
      ok = 0;
    }
    __builtin_amdgcn_s_sleep(4);
    *lds_flag = ok;
  }
  __syncthreads();
  const int ok = *lds_flag;
  __syncthreads();
  return ok != 0;
}

// Block-wide exclusive prefix sum of one int per thread (kThreads values).
// Within a wave: Kogge-Stone over 16-lane rows with DPP row shifts, then the
// row totals carried across rows with row broadcasts.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_add_src(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, false);
}
__device__ int block_exclusive_scan(int v, SHARED int* lds4, int* total) {
  const int lane = lane_id(), w = wave_id();
  int incl = v;
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xF, 0xF, true);   // row_shr:1
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xF, 0xF, true);   // row_shr:2
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xF, 0xF, true);   // row_shr:4
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xF, 0xF, true);   // row_shr:8
  incl += dpp_add_src<0x142, 0xA>(incl);                                 // row_bcast:15
  incl += dpp_add_src<0x143, 0xC>(incl);                                 // row_bcast:31
  if (lane == kWave - 1) lds4[w] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const int s = lds4[i];
    if (i < w) off += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return off + incl - v;
}

// ----------------------------------------------------------------------------
// Workgroup view of the routing (LDS), built once per workgroup
// ----------------------------------------------------------------------------
struct Lds {
  SHARED unsigned long long* bm;  // [E][nch] row bitmap of each expert
  SHARED int* cp;                 // [E][nch] rows of the expert in earlier chunks
  SHARED int* cnt;                // [E] rows per expert
  SHARED int* base;               // [E] first scratch row of the expert
  SHARED int* nmrb;               // [E+1] prefix of M-ranges per expert
  SHARED int* mrlist;             // [n_mr] expert of each routed M-range
  SHARED int16_t* rows;           // [T*K] scratch row -> token, grouped by expert
  SHARED int16_t* tki;            // [T][K] selected experts
  SHARED int16_t* prow;           // [T][K] scratch row of each pair (its expert output row)
  SHARED float* tkw;              // [T][K] their weights
  SHARED float* red;              // partial sums of the 4 waves
  SHARED int* misc;               // [0] n_mr, [1] flag, [3..7) scan scratch, [8..12) block_any,
                                  // [2] claimed item, [12..14) end of the last wait (thread 0),
                                  // [14] polling rounds of the last gather (thread 0),
                                  // [16..22) ends of a gather's first rounds (timeline)
  SHARED uint32_t* tks;           // [kThreads] one scratch word per thread (gather sink)
  SHARED uint16_t* xs;            // [T][xs_stride] the layer input (small batches)
  SHARED uint16_t* hs;            // [16][hs_stride] h rows of the current down item
  SHARED float* lg;               // [T][E] router logits (small batches)
  uint32_t epoch;                 // this run's tag
  int* ctr;                       // this run's counter block
};

__device__ Lds lds_view(KParams& p, SHARED char* smem) {
  Lds L;
  L.bm = (SHARED unsigned long long*)(smem + p.lds_bm);
  L.cp = (SHARED int*)(smem + p.lds_cp);
  L.cnt = (SHARED int*)(smem + p.lds_cnt);
  L.base = (SHARED int*)(smem + p.lds_base);
  L.nmrb = (SHARED int*)(smem + p.lds_nmrb);
  L.mrlist = (SHARED int*)(smem + p.lds_mrlist);
  L.rows = (SHARED int16_t*)(smem + p.lds_rows);
  L.tki = (SHARED int16_t*)(smem + p.lds_tki);
  L.prow = (SHARED int16_t*)(smem + p.lds_prow);
  L.tkw = (SHARED float*)(smem + p.lds_tkw);
  L.red = (SHARED float*)(smem + p.lds_red);
  L.misc = (SHARED int*)(smem + p.lds_misc);
  L.tks = (SHARED uint32_t*)(smem + p.lds_tks);
  L.xs = (SHARED uint16_t*)(smem + p.lds_xs);
  L.hs = (SHARED uint16_t*)(smem + p.lds_hs);
  L.lg = (SHARED float*)(smem + p.lds_lg);
  return L;
}

// Gather the words i < n with want(i) of this run with the whole workgroup:
// take(i, payload) is called for every such i whose word carries the current
// epoch (possibly more than once); stale words are read again, round by
// round, until none is.  kBatch loads per thread are in flight before any is
// examined.  false: the deadline passed or another workgroup reported an
// error.
template <typename LoadFn, typename TakeFn, typename WantFn>
__device__ __forceinline__ bool gather_tagged(KParams& p, const Lds& L, int n, LoadFn load, TakeFn take,
                                              WantFn want) {
  long long t_end = 0;
  // this thread's words still to take: bit kBatch j + b for word
  // tid + (kBatch j + b) kThreads of the first 8 batches; words past those
  // are all read again while any of them is stale
  unsigned long long todo = ~0ull;
  bool rest = true;
  int rounds = 0;
  while (true) {
    bool stale = false, rest_stale = false;
    int j = 0;
    for (int i0 = threadIdx.x; i0 < n; i0 += kBatch * kThreads, ++j) {
      const uint32_t m = j < 8 ? (uint32_t)(todo >> (kBatch * j)) & 0xffu : (rest ? 0xffu : 0u);
      uint64_t v[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int i = i0 + b * kThreads;
        v[b] = 0;
        if (i < n && (m >> b & 1u) && want(i)) v[b] = load(i);
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int i = i0 + b * kThreads;
        if (i < n && (m >> b & 1u) && want(i)) {
          if (tag_ok(v[b], L.epoch)) {
            take(i, (uint32_t)v[b]);
            if (j < 8) todo &= ~(1ull << (kBatch * j + b));
          } else {
            stale = true;
            rest_stale |= j >= 8;
          }
        }
      }
    }
    rest = rest_stale;
    if (p.trace && threadIdx.x == 0 && rounds < 3) ((SHARED long long*)(L.misc + 16))[rounds] = tl_clock(p);
    if (!block_any(stale, L.misc + 8)) break;
    if (!poll_round(p, &t_end, &rounds, L.misc + 1)) return false;
  }
  // when the gather ended and its rounds (read back by thread 0 for the timeline)
  if (threadIdx.x == 0) {
    *(SHARED long long*)(L.misc + 12) = tl_clock(p);
    L.misc[14] = rounds;
  }
  return true;
}
template <typename LoadFn, typename TakeFn>
__device__ __forceinline__ bool gather_tagged(KParams& p, const Lds& L, int n, LoadFn load, TakeFn take) {
  return gather_tagged(p, L, n, load, take, [](int) { return true; });
}

// The same for n <= kBatch kThreads words into LDS, without per-word
// branches: thread tid owns words tid + b kThreads; while any of them is
// missing it reloads all of them, and every word it examines is written,
// to slot(i) when wanted and current, else to the thread's own scratch word.
template <typename LoadFn, typename SlotFn, typename WantFn>
__device__ __forceinline__ bool gather_small(KParams& p, const Lds& L, int n, LoadFn load, SlotFn slot,
                                             WantFn want) {
  long long t_end = 0;
  int rounds = 0;
  uint32_t need = 0;                           // bit b: word b wanted, not yet taken
#pragma unroll
  for (int b = 0; b < kBatch; ++b) {
    const int i = threadIdx.x + b * kThreads;
    need |= (i < n && want(i)) ? 1u << b : 0u;
  }
  SHARED uint32_t* const sink = L.tks + threadIdx.x;
  while (true) {
    if (need != 0u) {
      uint64_t v[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) v[b] = load(min((int)threadIdx.x + b * kThreads, n - 1));
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const bool ok = (need >> b & 1u) && tag_ok(v[b], L.epoch);
        *(ok ? slot((int)threadIdx.x + b * kThreads) : sink) = (uint32_t)v[b];
        need &= ok ? ~(1u << b) : ~0u;
      }
    }
    if (p.trace && threadIdx.x == 0 && rounds < 3) ((SHARED long long*)(L.misc + 16))[rounds] = tl_clock(p);
    if (!block_any(need != 0u, L.misc + 8)) break;
    if (!poll_round(p, &t_end, &rounds, L.misc + 1)) return false;
  }
  if (threadIdx.x == 0) {
    *(SHARED long long*)(L.misc + 12) = tl_clock(p);
    L.misc[14] = rounds;
  }
  return true;
}

// Sort-free placement ("routing without sorting": each expert's rows go to
// 8-row tiles in row order, positions from a bitmap and population counts).
// Every pair (t, k) sets bit t of expert idx[t][k]'s bitmap; an expert's
// count is the popcount of its bitmap; a pair's rank is the popcount of the
// expert's bits below t.  Row r of expert e lives at scratch row base[e] + r.
// The bitmaps must be zero on entry (clear_placement, earlier, with a
// barrier in between).  One block scan yields both the rows and the 64-row
// ranges before each expert (packed 16 + 16 bits: T K <= 8192).
__device__ __forceinline__ void clear_placement(KParams& p, const Lds& L) {
  for (int i = threadIdx.x; i < p.E * p.nch; i += kThreads) L.bm[i] = 0ull;
}
__device__ __forceinline__ void build_placement(KParams& p, const Lds& L) {
  const int tid = threadIdx.x;
  const int E = p.E, nch = p.nch, n = p.T * p.K;
  // the pair loops take kPairBatch pairs per thread at a time, so their LDS
  // round trips overlap
  constexpr int kPairBatch = 4;
  for (int i0 = tid; i0 < n; i0 += kPairBatch * kThreads) {
    int e[kPairBatch], t[kPairBatch];
#pragma unroll
    for (int u = 0; u < kPairBatch; ++u) {
      const int i = min(i0 + u * kThreads, n - 1);
      e[u] = L.tki[i];
      t[u] = (int)fdiv((uint32_t)i, p.fd_k.m, p.fd_k.s);
    }
#pragma unroll
    for (int u = 0; u < kPairBatch; ++u)
      if (i0 + u * kThreads < n)
        __hip_atomic_fetch_or(&L.bm[e[u] * nch + (t[u] >> 6)], 1ull << (t[u] & 63), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  __syncthreads();
  int c = 0, nmr = 0;
  if (tid < E) {
    for (int ch = 0; ch < nch; ++ch) {
      L.cp[tid * nch + ch] = c;
      c += __popcll(L.bm[tid * nch + ch]);
    }
    nmr = (c + p.mrange - 1) / p.mrange;
  }
  int tot;
  const int packed = block_exclusive_scan(c | nmr << 16, L.misc + 3, &tot);
  const int base = packed & 0xffff, mrb = packed >> 16;
  if (tid < E) {
    L.cnt[tid] = c;
    L.base[tid] = base;
    L.nmrb[tid] = mrb;
    for (int j = 0; j < nmr; ++j) L.mrlist[mrb + j] = tid;
  }
  if (tid == 0) {
    L.nmrb[E] = tot >> 16;
    L.misc[0] = tot >> 16;
  }
  __syncthreads();
  for (int i0 = tid; i0 < n; i0 += kPairBatch * kThreads) {
    int e[kPairBatch], t[kPairBatch], r[kPairBatch];
#pragma unroll
    for (int u = 0; u < kPairBatch; ++u) {
      const int i = min(i0 + u * kThreads, n - 1);
      e[u] = L.tki[i];
      t[u] = (int)fdiv((uint32_t)i, p.fd_k.m, p.fd_k.s);
    }
#pragma unroll
    for (int u = 0; u < kPairBatch; ++u) {
      const unsigned long long below = L.bm[e[u] * nch + (t[u] >> 6)] & ((1ull << (t[u] & 63)) - 1ull);
      r[u] = L.base[e[u]] + L.cp[e[u] * nch + (t[u] >> 6)] + __popcll(below);
    }
#pragma unroll
    for (int u = 0; u < kPairBatch; ++u) {
      const int i = i0 + u * kThreads;
      if (i < n) {
        L.rows[r[u]] = (int16_t)t[u];
        L.prow[i] = (int16_t)r[u];
      }
    }
  }
  __syncthreads();
}

__device__ __forceinline__ int pair_rank(KParams& p, const Lds& L, int t, int e) {
  const unsigned long long below = L.bm[e * p.nch + (t >> 6)] & ((1ull << (t & 63)) - 1ull);
  return L.cp[e * p.nch + (t >> 6)] + __popcll(below);
}

// Optional debug copies of routing and placement (written by workgroup 0).
__device__ __forceinline__ void write_routing_debug(KParams& p, const Lds& L) {
  for (int i = threadIdx.x; i < p.T * p.K; i += kThreads) {
    if (p.dbg_idx) st(p.dbg_idx + i, (int)L.tki[i]);
    if (p.dbg_w) st(p.dbg_w + i, L.tkw[i]);
    if (p.dbg_rank) st(p.dbg_rank + i, pair_rank(p, L, i / p.K, L.tki[i]));
  }
  if (p.dbg_count)
    for (int e = threadIdx.x; e < p.E; e += kThreads) st(p.dbg_count + e, L.cnt[e]);
}

// ----------------------------------------------------------------------------
// Router: logits of expert e for up to 8 rows; the 4 waves split H.  x comes
// from LDS when the batch is small enough to keep it there.
// ----------------------------------------------------------------------------
// Router tile (batches above 16 rows): logits of rows [16 rt, +16) x experts
// [16 et, +16) with v_mfma_f32_16x16x4_f32; the 4 waves split H.  Lane l =
// (n, kq), n = l % 16, kq = l / 16, loads 4 consecutive K of row n of x and
// of expert n's router row; its i-th value feeds the i-th of 4 MFMAs, so the
// 4 instructions together cover 16 consecutive K (any split of a sum's terms
// over the instructions gives the same sum up to rounding order).  The fp32
// partial tiles of the waves are added in LDS in wave order.
__device__ __forceinline__ void router_tile_item(KParams& p, const Lds& L, int item) {
  const int w = wave_id(), lane = lane_id();
  const int n = lane & 15, kq = lane >> 4;
  const int n_et = (p.E + kRouterTile - 1) / kRouterTile;
  const int tile = item / p.router_ks, ks = item % p.router_ks;
  const int t0 = (tile / n_et) * kRouterTile, e0 = (tile % n_et) * kRouterTile;
  const int nt = min(kRouterTile, p.T - t0), ne = min(kRouterTile, p.E - e0);
  const int kw = p.H / p.router_ks / kWaves;   // K per wave (a multiple of 16)
  const int kbase = ks * (p.H / p.router_ks) + w * kw;
  const uint16_t* xr = p.x + (size_t)(t0 + min(n, nt - 1)) * p.H + kbase + 4 * kq;
  // the router rows come from their tiled copy: one step of 16 K of the 16
  // experts is one contiguous KiB, lane (n, kq) holding expert n's K 4 kq .. + 3
  const f32x4* wr = p.router_wt + ((size_t)(e0 / kRouterTile) * (p.H / 16) + kbase / 16) * kWave + lane;
  // the bias goes with part 0 (the top-k items add the parts in order); it
  // is requested first, so its round trip overlaps the weights'
  const float bv = ld(p.router_b + e0 + min(n, ne - 1));   // unconditional: no branch, no early wait
  const float bias = (ks == 0 && p.has_bias && w == 0 && n < ne) ? bv : 0.f;
  // one accumulator per MFMA slot i, so consecutive MFMAs do not depend on
  // each other; the four are added in a fixed order at the end
  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // two register stages of kU 16-K steps each, loaded a stage ahead
  constexpr int kU = 8;
  struct Stage { u32x2 xa[kU]; f32x4 wb[kU]; };
  auto load = [&](Stage& S, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int k = min(k0 + 16 * u, kw - 16);  // past the end: reread the last step (unused)
      S.xa[u] = ld((const u32x2*)(xr + k));
      S.wb[u] = ld(wr + (size_t)(k / 16) * kWave);
    }
  };
  auto compute = [&](const Stage& S, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (k0 + 16 * u < kw) {
        acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf16_to_f32(S.xa[u].x & 0xffffu), S.wb[u].x, acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf16_to_f32(S.xa[u].x >> 16), S.wb[u].y, acc[1], 0, 0, 0);
        acc[2] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf16_to_f32(S.xa[u].y & 0xffffu), S.wb[u].z, acc[2], 0, 0, 0);
        acc[3] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf16_to_f32(S.xa[u].y >> 16), S.wb[u].w, acc[3], 0, 0, 0);
      }
    }
  };
  constexpr int kStep = 16 * kU;
  Stage A, B;
  load(A, 0);
  for (int k0 = 0; k0 < kw; k0 += 2 * kStep) {
    if (k0 + kStep < kw) load(B, k0 + kStep);
    compute(A, k0);
    if (k0 + 2 * kStep < kw) load(A, k0 + 2 * kStep);
    if (k0 + kStep < kw) compute(B, k0 + kStep);
  }
  // D layout: lane l holds rows 4 kq + i (x rows) of column n (expert)
  SHARED f32x4* part = (SHARED f32x4*)L.red;   // [kWaves][64]
  part[w * kWave + lane] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();
  if (w == 0) {
    f32x4 s = part[lane];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) s += part[ww * kWave + lane];
    uint64_t* out = p.lgt + (size_t)ks * p.T * p.E;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * kq + i;
      if (r < nt && n < ne) st_tag(out + (size_t)(t0 + r) * p.E + e0 + n, __float_as_uint(s[i] + bias), L.epoch);
    }
  }
  __syncthreads();                             // the partials area is free again
}

// With stage_x (the item covers every row), the x values it loads are also
// written to the workgroup's LDS copy of x, which later items read.
// Returns (timeline only) when this workgroup's partial sums were complete.
// NORM (pre-norm block runs): x is xn; the first pass's weights are
// requested before the wait for the item's rows.  LLONG_MIN: the wait failed.
__device__ bool wait_rows(KParams& p, const Lds& L, int t0, int n);
struct NoHook {
  __device__ void operator()() const {}
};
template <bool NORM = false, class Pre = NoHook, class Post = NoHook>
__device__ __forceinline__ long long router_item(KParams& p, const Lds& L, int item, bool stage_x,
                                                 Pre&& pre_barrier = Pre{}, Post&& post_barrier = Post{}) {
  const int w = wave_id(), lane = lane_id();
  const int e = item % p.E;
  const int t0 = (item / p.E) * kRouterRows;
  const int nt = min(kRouterRows, p.T - t0);
  const int n16 = p.H / 16;                    // 16-element chunks
  // the bias is requested first, so its round trip overlaps the weights'
  const float bv = ld(p.router_b + e);        // unconditional: no branch, no early wait
  const float bias = p.has_bias ? bv : 0.f;
  float acc[kRouterRows];
#pragma unroll
  for (int j = 0; j < kRouterRows; ++j) acc[j] = 0.f;
  const f32x4* wr = (const f32x4*)(p.router_w + (size_t)e * p.H);
  const u32x4* xg[kRouterRows];                // rows past nt reread the last row
#pragma unroll
  for (int j = 0; j < kRouterRows; ++j) xg[j] = (const u32x4*)(p.x + (size_t)(t0 + min(j, nt - 1)) * p.H);
  // each thread owns 16 consecutive elements per pass; a pass issues all of
  // its loads (4 x 16 B of weights, 2 x 16 B per row) before the first use
  for (int c0 = 0; c0 < n16; c0 += kThreads) {
    const int c = min(c0 + (int)threadIdx.x, n16 - 1);
    const bool live = c0 + (int)threadIdx.x < n16;
    f32x4 wv[4];
    u32x4 xv[kRouterRows][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[i] = ld(wr + 4 * c + i);
    if constexpr (NORM) {
      if (c0 == 0 && !wait_rows(p, L, t0, nt)) return LLONG_MIN;
    }
#pragma unroll
    for (int j = 0; j < kRouterRows; ++j) {
      xv[j][0] = ld(xg[j] + 2 * c);
      xv[j][1] = ld(xg[j] + 2 * c + 1);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      wv[i] = live ? wv[i] : z;
    }
    if (stage_x && live) {
#pragma unroll
      for (int j = 0; j < kRouterRows; ++j) {
        if (j < nt) {
          SHARED u32x4* d = (SHARED u32x4*)(L.xs + (size_t)j * p.xs_stride + 16 * c);
          d[0] = xv[j][0];
          d[1] = xv[j][1];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kRouterRows; ++j) {
      float a = acc[j];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 xw = xv[j][h];
        const f32x4 w0 = wv[2 * h], w1 = wv[2 * h + 1];
        a += w0.x * bf16_to_f32(xw.x & 0xffffu) + w0.y * bf16_to_f32(xw.x >> 16) +
             w0.z * bf16_to_f32(xw.y & 0xffffu) + w0.w * bf16_to_f32(xw.y >> 16);
        a += w1.x * bf16_to_f32(xw.z & 0xffffu) + w1.y * bf16_to_f32(xw.z >> 16) +
             w1.z * bf16_to_f32(xw.w & 0xffffu) + w1.w * bf16_to_f32(xw.w >> 16);
      }
      acc[j] = a;
    }
  }
#pragma unroll
  for (int j = 0; j < kRouterRows; ++j) asm volatile("" ::"v"(acc[j]));
  const long long t_sums = tl_clock(p);
  SHARED float* part = L.red;                  // [kWaves][8]
#pragma unroll
  for (int j = 0; j < kRouterRows; ++j) {
    const float s = wave_sum(acc[j]);
    if (lane == 0) part[w * kRouterRows + j] = s;
  }
  pre_barrier();                               // (the run's arrival, when it is still to be read)
  __syncthreads();
  post_barrier();
  // wave 0, lane 8 c + j: row j's logit, stored as copy c (every copy and row
  // in one store instruction)
  static_assert(kLgCopies * kRouterRows == kWave, "one lane per (copy, row)");
  if (w == 0) {
    const int j = lane % kRouterRows, c = lane / kRouterRows;
    float s = part[j];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) s += part[ww * kRouterRows + j];
    s += bias;
    if (j < nt && c < p.lg_copies)
      st_tag(p.lgt + (((size_t)c * p.E + e) << p.lg_tp_log2) + t0 + j, __float_as_uint(s), L.epoch);
    if (j < nt && c == 0 && p.dbg_logits) st(p.dbg_logits + (size_t)(t0 + j) * p.E + e, s);
  }
  __syncthreads();                             // the partials area is free again
  return t_sums;
}

// ----------------------------------------------------------------------------
// Top-k of a row in one wave.  Lane l holds experts 4l .. 4l+3 as
// order-preserving unsigned keys of their logits (ranking by logit equals
// ranking by sigmoid score).  K rounds each take the wave maximum key and,
// among its holders, the lowest expert id (the lowest lane, then its lowest
// slot), then retire it: the picks come out in (score desc, id asc) order.
// Weights: sigmoid of the selected logits over their sum.
// ----------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_ukey(float v) {
  // NaN maps to 1, just above absent and retired experts (0), so it never
  // displaces a score
  if (v != v) return 1u;
  const int b = __float_as_int(v);
  const int k = b >= 0 ? b : (b ^ 0x7fffffff);
  return (uint32_t)k ^ 0x80000000u;
}
__device__ __forceinline__ float ukey_value(uint32_t u) {
  const int k = (int)(u ^ 0x80000000u);
  return __int_as_float(k >= 0 ? k : (k ^ 0x7fffffff));
}
// Maximum / minimum over the 64 lanes, returned in every lane, all in vector
// registers: DPP within each 16-lane row, then the gfx950 lane swaps across
// rows (32 apart, then 16 apart).  No scalar register carries the result, so
// independent reductions of one wave overlap.
__device__ __forceinline__ uint32_t wave_max_v(uint32_t v) {
  v = max(v, dpp<kDppXor1>(v));
  v = max(v, dpp<kDppXor2>(v));
  v = max(v, dpp<kDppHalfMirror>(v));
  v = max(v, dpp<kDppMirror>(v));
  const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = max(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max(b[0], b[1]);
}
__device__ __forceinline__ uint32_t wave_min_v(uint32_t v) {
  v = min(v, dpp<kDppXor1>(v));
  v = min(v, dpp<kDppXor2>(v));
  v = min(v, dpp<kDppHalfMirror>(v));
  v = min(v, dpp<kDppMirror>(v));
  const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = min(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return min(b[0], b[1]);
}

// Top-k of NR rows at once in one wave (their rounds interleave).  Row r's
// logits are lg[t[r]][0..E) in LDS.  Returns, in lanes k < K, row r's k-th
// expert and weight.
template <int NR>
__device__ __forceinline__ void topk_rows(KParams& p, const SHARED float* lg, const int (&t)[NR],
                                          int (&out_e)[NR], float (&out_w)[NR]) {
  const uint32_t lane = lane_id();
  const int K = p.K;
  uint32_t uk[NR][4];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      const float v = lg[t[r] * p.E + min(e, p.E - 1)];
      uk[r][j] = e < p.E ? order_ukey(v) : 0u;
    }
  uint32_t sel_k[NR], sel_e[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) sel_k[r] = sel_e[r] = 0;
  for (int k = 0; k < K; ++k) {
    uint32_t M[NR], W[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const uint32_t m = max(max(uk[r][0], uk[r][1]), max(uk[r][2], uk[r][3]));
      M[r] = wave_max_v(m);
      // lowest expert id holding the maximum: ids 4 lane + j grow with lane, then j
      const uint32_t fj = uk[r][0] == M[r] ? 0u : uk[r][1] == M[r] ? 1u : uk[r][2] == M[r] ? 2u : 3u;
      W[r] = wave_min_v(m == M[r] ? 4 * lane + fj : 0xffffu);
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      sel_k[r] = lane == (uint32_t)k ? M[r] : sel_k[r];
      sel_e[r] = lane == (uint32_t)k ? W[r] : sel_e[r];
#pragma unroll
      for (int j = 0; j < 4; ++j) uk[r][j] = 4 * lane + j == W[r] ? 0u : uk[r][j];
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const float s = (int)lane < K ? 1.0f / (1.0f + __expf(-ukey_value(sel_k[r]))) : 0.f;
    const float sum = wave_sum(s);
    out_e[r] = (int)sel_e[r];
    out_w[r] = s / sum;
  }
}

// Maximum over each 32-lane half of the wave (lanes 0-31 and 32-63
// separately), returned in every lane of the half: DPP within each 16-lane
// row, then the gfx950 16-lane swap between the rows of a half.
__device__ __forceinline__ uint32_t half_max_v(uint32_t v) {
  v = max(v, dpp<kDppXor1>(v));
  v = max(v, dpp<kDppXor2>(v));
  v = max(v, dpp<kDppHalfMirror>(v));
  v = max(v, dpp<kDppMirror>(v));
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max(b[0], b[1]);
}
__device__ __forceinline__ float half_sum_v(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Keys of experts 8 hl .. 8 hl + 7 of row t (lane hl of a half): read as two
// 16-byte LDS words when the row allows (E a multiple of 4), all reads issued
// before any key is formed, absent experts (id >= E) keyed 0.
__device__ __forceinline__ void load_keys8(KParams& p, const SHARED float* lg, int t, uint32_t hl, uint32_t (&uk)[8]) {
  float v[8];
  const int e0 = 8 * (int)hl;
  if ((p.E & 3) == 0 && e0 + 8 <= p.E) {
    const SHARED f32x4* q = (const SHARED f32x4*)(lg + t * p.E + e0);
    const f32x4 a = q[0], b = q[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = lg[t * p.E + min(e0 + j, p.E - 1)];
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t k = order_ukey(v[j]);
    uk[j] = e0 + j < p.E ? k : 0u;
  }
}

// Address translations of the expert weights, warmed while the routing is
// computed (the first items of every expert would otherwise each wait for
// page-table walks on an otherwise idle memory system).  The n workgroups
// that have no router or shared item each read one word from every n/8-th
// 2 MiB page, a thread per page; workgroup i's share goes to compute-unit
// group i mod 8, which is where consecutive workgroups are placed.
constexpr size_t kPageBytes = size_t(1) << 21;
__device__ __forceinline__ uint32_t touch_weight_pages(KParams& p, int i, int n) {
  const int per = n / 8, r = i / 8;
  if (per < 1 || r >= per) return 0;
  const size_t b13 = p.w13_bytes, b2 = p.w2_bytes, bs13 = p.s13_bytes, bs2 = p.s2_bytes;
  const size_t n13 = (b13 + kPageBytes - 1) / kPageBytes, n2 = (b2 + kPageBytes - 1) / kPageBytes;
  const size_t ns13 = (bs13 + kPageBytes - 1) / kPageBytes, ns2 = (bs2 + kPageBytes - 1) / kPageBytes;
  uint32_t acc = 0;
  for (size_t j = r + (size_t)threadIdx.x * per; j < n13 + n2 + ns13 + ns2; j += (size_t)kThreads * per) {
    const char* a;
    if (j < n13) a = (const char*)p.w13p + j * kPageBytes;
    else if (j < n13 + n2) a = (const char*)p.w2p + (j - n13) * kPageBytes;
    else if (j < n13 + n2 + ns13) a = (const char*)p.s13p + (j - n13 - n2) * kPageBytes;
    else a = (const char*)p.s2p + (j - n13 - n2 - ns13) * kPageBytes;
    acc += *(const volatile GLOBAL uint32_t*)a;
  }
  return acc;
}

// Top-k of two rows in one wave, one per 32-lane half: lane l of half h
// holds experts 8 (l % 32) .. 8 (l % 32) + 7 of row t[h] as order-preserving
// keys, first sorted within the lane (keys descending; the sort is stable,
// so equal keys keep ascending ids).  Each of the K rounds takes the half's
// maximum head key; its lowest holder lane (lanes hold ascending id ranges)
// gives the pick's id and pops its head, so both rows share every
// reduction and the picks come out in (score desc, id asc) order.  Returns,
// in lanes k < K of each half, that half's row's k-th expert and weight.
__device__ __forceinline__ void topk_pair(KParams& p, const SHARED float* lg, int tA, int tB, int* out_e,
                                          float* out_w) {
  const uint32_t hl = lane_id() & 31;
  const bool lo = lane_id() < 32;
  const int t = lo ? tA : tB;
  const int K = p.K;
  uint32_t uk[8], ui[8];
  load_keys8(p, lg, t, hl, uk);
#pragma unroll
  for (int j = 0; j < 8; ++j) ui[j] = 8 * hl + j;
  // odd-even transposition sort: adjacent exchanges on strictly greater keys
#pragma unroll
  for (int r = 0; r < 8; ++r) {
#pragma unroll
    for (int j = r & 1; j + 1 < 8; j += 2) {
      const bool sw = uk[j + 1] > uk[j];
      const uint32_t k0 = sw ? uk[j + 1] : uk[j], k1 = sw ? uk[j] : uk[j + 1];
      const uint32_t i0 = sw ? ui[j + 1] : ui[j], i1 = sw ? ui[j] : ui[j + 1];
      uk[j] = k0;
      uk[j + 1] = k1;
      ui[j] = i0;
      ui[j + 1] = i1;
    }
  }
  uint32_t sel_k = 0, sel_e = 0;
  for (int k = 0; k < K; ++k) {
    const uint32_t M = half_max_v(uk[0]);
    const unsigned long long bal = __ballot(uk[0] == M);
    // each half holds its own maximum, so both halves of the ballot are
    // nonzero; both picks are read and selected per lane (no branch)
    const int wlo = __builtin_ctz((uint32_t)bal), whi = 32 + __builtin_ctz((uint32_t)(bal >> 32));
    const uint32_t Wlo = __builtin_amdgcn_readlane(ui[0], wlo), Whi = __builtin_amdgcn_readlane(ui[0], whi);
    const uint32_t W = lo ? Wlo : Whi;
    sel_k = hl == (uint32_t)k ? M : sel_k;
    sel_e = hl == (uint32_t)k ? W : sel_e;
    const bool win = (int)lane_id() == (lo ? wlo : whi);
#pragma unroll
    for (int j = 0; j < 7; ++j) {
      uk[j] = win ? uk[j + 1] : uk[j];
      ui[j] = win ? ui[j + 1] : ui[j];
    }
    uk[7] = win ? 0u : uk[7];
  }
  const float s = (int)hl < K ? 1.0f / (1.0f + __expf(-ukey_value(sel_k))) : 0.f;
  const float sum = half_sum_v(s);
  *out_e = (int)sel_e;
  *out_w = s / sum;
}

// This run's router logits (this workgroup's copy, [E][lg_tp] tagged words)
// into LDS lg as [T][E], once every one of them carries the current epoch.
__device__ __forceinline__ bool gather_logits(KParams& p, const Lds& L) {
  const int c = blockIdx.x % p.lg_copies;
  const int sh = p.lg_tp_log2, mask = (1 << sh) - 1;
  const uint64_t* src = p.lgt + ((size_t)c * p.E << sh);
  auto load = [&](int i) { return ld_tag(src + i); };
  auto want = [&](int i) { return (i & mask) < p.T; };
  if ((p.E << sh) <= kBatch * kThreads)
    return gather_small(p, L, p.E << sh, load,
                        [&](int i) { return (SHARED uint32_t*)L.lg + (i & mask) * p.E + (i >> sh); }, want);
  return gather_tagged(
      p, L, p.E << sh, load, [&](int i, uint32_t v) { L.lg[(i & mask) * p.E + (i >> sh)] = __uint_as_float(v); },
      want);
}

// A top-k item's partial logits: KS parts of its nt x E logits (part k of row
// t0 + r at lgt[k T E + (t0 + r) E .. + E)) into LDS lg[k per_part + j],
// per_part = nt E.  Thread tid owns words j = tid + b kThreads of every part:
// at most kRouterKsMax x 4 of them (per_part <= kWaves E <= 4 kThreads), all
// requested at once at fixed offsets from one base per part, with no
// per-word division (parts past router_ks are skipped by a uniform branch,
// so no dummy address is read by every thread: one hot line slows every
// stream on its channel).  A position past the item's words (E < 256, or the
// last item's fewer rows) reads the part's last word of the item and is
// written to the thread's own scratch word.  While any word is stale all are
// read again, round by round.
__device__ __forceinline__ bool gather_topk_parts(KParams& p, const Lds& L, int t0, int per_part) {
  constexpr int kJ = kWaves * kMaxExperts / kThreads;   // words per thread and part
  const int KS = p.router_ks;
  const size_t part = (size_t)p.T * p.E;
  const uint64_t* const rows = p.lgt + (size_t)t0 * p.E;   // part 0 of the item's rows
  SHARED uint32_t* const sink = L.tks + threadIdx.x;
  long long t_end = 0;
  int rounds = 0;
  while (true) {
    uint64_t v[kRouterKsMax][kJ];
#pragma unroll
    for (int k = 0; k < kRouterKsMax; ++k) {
      if (k < KS) {                            // uniform
        const uint64_t* const src = rows + k * part;
#pragma unroll
        for (int b = 0; b < kJ; ++b) v[k][b] = ld_tag(src + min((int)threadIdx.x + b * kThreads, per_part - 1));
      }
    }
    bool stale = false;
#pragma unroll
    for (int k = 0; k < kRouterKsMax; ++k) {
      if (k < KS) {
#pragma unroll
        for (int b = 0; b < kJ; ++b) {
          const int j = (int)threadIdx.x + b * kThreads;
          const bool in = j < per_part;
          const bool ok = in && tag_ok(v[k][b], L.epoch);
          *(ok ? (SHARED uint32_t*)L.lg + k * per_part + j : sink) = (uint32_t)v[k][b];
          stale |= in && !ok;
        }
      }
    }
    if (p.trace && threadIdx.x == 0 && rounds < 3) ((SHARED long long*)(L.misc + 16))[rounds] = tl_clock(p);
    if (!block_any(stale, L.misc + 8)) break;
    if (!poll_round(p, &t_end, &rounds, L.misc + 1)) return false;
  }
  if (threadIdx.x == 0) {
    *(SHARED long long*)(L.misc + 12) = tl_clock(p);
    L.misc[14] = rounds;
  }
  return true;
}

// Distributed top-k item (large batches): rows 4 item .. 4 item + 3, one per
// wave, to global memory.  The logits arrive as router_ks partial sums
// (gathered as [ks][row][E]) and are added in ks order.
__device__ __forceinline__ bool topk_item(KParams& p, const Lds& L, int item) {
  const int t0 = item * kWaves;
  const int nt = min(kWaves, p.T - t0);
  const int KS = p.router_ks;
  const int per_part = nt * p.E;
  __syncthreads();                             // earlier readers of the lg area are done
  if (!gather_topk_parts(p, L, t0, per_part)) return false;
  __syncthreads();
  for (int i = threadIdx.x; i < per_part; i += kThreads) {
    float v = L.lg[i];
    for (int k = 1; k < KS; ++k) v += L.lg[k * per_part + i];
    L.lg[i] = v;
    if (p.dbg_logits) st(p.dbg_logits + (size_t)t0 * p.E + i, v);
  }
  __syncthreads();
  const int w = wave_id();
  if (w < nt) {
    const int tr[1] = {w};
    int e[1];
    float wk[1];
    topk_rows<1>(p, L.lg, tr, e, wk);
    if (lane_id() < p.K) {
      st_coh(p.topk_idx + (t0 + w) * p.K + lane_id(), e[0]);
      st_coh(p.topk_w + (t0 + w) * p.K + lane_id(), wk[0]);
    }
  }
  return true;
}

// A down item's h rows (nrows x I bf16, written by other workgroups) into
// LDS, once each word carries this run's epoch.
__device__ __forceinline__ bool stage_h_rows(KParams& p, const Lds& L, int row0, int nrows) {
  const int per_row = p.I / 2;                // tagged words per row
  const uint64_t* src = p.h_scr + (size_t)row0 * per_row;
  auto slot = [&](int i) {
    const int r = (int)fdiv((uint32_t)i, p.fd_h2.m, p.fd_h2.s);
    return (SHARED uint32_t*)(L.hs + (size_t)r * p.hs_stride + 2 * (i - r * per_row));
  };
  if (nrows * per_row <= kBatch * kThreads)
    return gather_small(p, L, nrows * per_row, [&](int i) { return ld_tag(src + i); }, slot,
                        [](int) { return true; });
  return gather_tagged(p, L, nrows * per_row, [&](int i) { return ld_tag(src + i); },
                       [&](int i, uint32_t v) { *slot(i) = v; });
}

// Wait until every word of h rows [row0, row0 + nrows) carries this run's
// epoch (down items that read h straight from global memory).
__device__ __forceinline__ bool verify_h_rows(KParams& p, const Lds& L, int row0, int nrows) {
  const int per_row = p.I / 2;
  return gather_tagged(p, L, nrows * per_row, [&](int i) { return ld_tag(p.h_scr + (size_t)row0 * per_row + i); },
                       [&](int, uint32_t) {});
}

// 8 consecutive bf16 of a tagged h row (4 words): the payload halves.
__device__ __forceinline__ u32x4 ld_h8(const uint64_t* w) {
  const u32x4 a = ld_coh16(w), b = ld_coh16(w + 2);
  return (u32x4){a.x, a.z, b.x, b.z};
}

// ----------------------------------------------------------------------------
// Down-wave epilogue: each wave stores its output rows as tagged words and
// counts itself in for its 128-column group (no wait for the stores).
// ----------------------------------------------------------------------------
__device__ __forceinline__ int down_waves_in_group(KParams& p, int rg) {
  if (p.wide) return 1;                       // a wide down wave covers a whole group
  const int nc = min(kDownRows, p.H - rg * kDownRows);
  return min(kWaves, (nc + 2 * kTileRows - 1) / (2 * kTileRows));
}

// ----------------------------------------------------------------------------
// Combine item: rows [R rc, R rc + R) x columns [128 rg, 128 rg + 128) of
//   y[t] = bf16( o_shared[t] + sum_k w[t][k] o_{idx[t][k]}[t] ),
// summed in exactly that order, once every down wave of column group rg has
// counted in and every expert output read carries this run's epoch.  Each
// thread computes kOut outputs (R = 2 kOut rows per item) from up to kIn
// inputs each (K <= kIn - 1 routed ones, the shared one last).  RES (pre-norm
// block runs): y[t] = bf16( x_in[t] + that sum ), the residual added to the
// unrounded sum.
// ----------------------------------------------------------------------------
template <int kOut, int kIn, bool RES = false>
__device__ __forceinline__ bool combine_item(KParams& p, const Lds& L, int rc, int rg, int n_mr) {
  constexpr int kRows = kOut * kThreads / kDownRows;
  constexpr int kSh = kIn - 1;                                // slot of the shared input
  const int K = p.K;
  const int c0 = rg * kDownRows;
  const int nc = min(kDownRows, p.H - c0);
  const int t0 = rc * kRows;
  const int nt = min(kRows, p.T - t0);
  long long t_end = 0;
  int rounds = 0;
  // Many combine items (large batches) first wait for the column group's
  // count, so they do not poll expert outputs that are still far from done;
  // a few items poll the outputs' tags directly, re-reading only stale words.
  if (p.n_cmb > 128) {
    const int target = (n_mr + p.n_mr_sh) * down_waves_in_group(p, rg);
    if (!wait_geq(p, L.ctr + kCtrRgDone + rg * kLine, target, L.misc + 1)) return false;
  }
  int tt[kOut];
  bool live[kOut];
  const uint64_t* src[kOut];
#pragma unroll
  for (int j = 0; j < kOut; ++j) {
    const int o = threadIdx.x + kThreads * j;
    const int r = o / kDownRows, c = o % kDownRows;
    live[j] = r < nt && c < nc;
    tt[j] = t0 + min(r, nt - 1);
    src[j] = p.o_scr + c0 + min(c, nc - 1);
  }
  // the residual, requested before the outputs are polled
  uint32_t res[kOut];
  if constexpr (RES) {
#pragma unroll
    for (int j = 0; j < kOut; ++j) {
      const int o = threadIdx.x + kThreads * j;
      res[j] = ld(p.x_in + (size_t)tt[j] * p.H + c0 + min(o % kDownRows, nc - 1));
    }
  }
  // scratch row of every input: the K routed outputs, then the shared one
  int row[kOut][kIn];
#pragma unroll
  for (int j = 0; j < kOut; ++j)
#pragma unroll
    for (int k = 0; k < kIn; ++k)
      row[j][k] = k == kSh ? p.T * K + tt[j] : (k < K ? L.prow[tt[j] * K + k] : 0);
  // A thread missing any of its inputs reads all of them again (no
  // per-word branches; the conditions on k are uniform).
  uint64_t v[kOut][kIn];
  const uint64_t fresh = (uint64_t)L.epoch << 32;   // tag-only stand-in for a missing shared expert
#pragma unroll
  for (int j = 0; j < kOut; ++j)
#pragma unroll
    for (int k = 0; k < kIn; ++k) v[j][k] = fresh;
  bool need = true;
  while (true) {
    if (need) {
#pragma unroll
      for (int j = 0; j < kOut; ++j)
#pragma unroll
        for (int k = 0; k < kIn; ++k)
          if ((k < K && k < kSh) || (k == kSh && p.S)) v[j][k] = ld_tag(src[j] + (size_t)row[j][k] * p.H);
      need = false;
#pragma unroll
      for (int j = 0; j < kOut; ++j)
#pragma unroll
        for (int k = 0; k < kIn; ++k) need |= live[j] && !tag_ok(v[j][k], L.epoch);
    }
    if (!block_any(need, L.misc + 8)) break;
    if (!poll_round(p, &t_end, &rounds, L.misc + 1)) return false;
  }
#pragma unroll
  for (int j = 0; j < kOut; ++j) {
    float acc = p.S ? __uint_as_float((uint32_t)v[j][kSh]) : 0.f;
#pragma unroll
    for (int k = 0; k < kSh; ++k)
      if (k < K) acc += L.tkw[tt[j] * K + k] * __uint_as_float((uint32_t)v[j][k]);
    if constexpr (RES) acc = bf16_to_f32(res[j]) + acc;
    const int o = threadIdx.x + kThreads * j;
    if (live[j]) st(p.y + (size_t)tt[j] * p.H + c0 + o % kDownRows, f32_to_bf16(acc));
  }
  if (threadIdx.x == 0) *(SHARED long long*)(L.misc + 12) = tl_clock(p);   // timeline
  return true;
}

// ----------------------------------------------------------------------------
// Gate/up epilogue of element i of every lane's four values of a 16x16
// gate/up result: column n < 8 is gate row 8 rb + n, column n + 8 the
// matching up row, result row 4 kq + i (block-relative; rows from nrows on
// are not stored).  h = bf16(silu(min(g, L)) * clamp(u, -L, L)) goes out as
// tagged pairs of adjacent columns (lanes with even n < 8).  All lanes of
// the wave take part (the DPP reads cross lanes).
__device__ __forceinline__ void swiglu_out(KParams& p, const Lds& L, float s, int i, int sbase, int r0, int nrows,
                                           int rb) {
  const int lane = lane_id(), n = lane & 15, kq = lane >> 4;
  const float g = s;
  const float u = dpp<kDppRowRor8>(s);
  const float gc = fminf(g, p.swiglu_limit), uc = fminf(fmaxf(u, -p.swiglu_limit), p.swiglu_limit);
  const uint32_t hb = f32_to_bf16(gc * __builtin_amdgcn_rcpf(1.0f + __expf(-gc)) * uc);
  const uint32_t hb_next = dpp<kDppRowShl1>(hb);             // column n + 1
  const int r = 4 * kq + i;
  if (n < 8 && (n & 1) == 0 && r < nrows)
    st_tag(p.h_scr + (size_t)(sbase + r0 + r) * (p.I / 2) + (8 * rb + n) / 2, hb | (hb_next << 16), L.epoch);
}

// Expert gate/up: one 16-row block (8 gate rows + 8 up rows) of one expert for
// up to 64 of its rows.  The 4 waves split the H/64 tiles (wave w takes tiles
// w, w+4, ...); weight loads run up to two stages ahead of the MFMAs; partial
// sums meet in LDS; then h = bf16(silu(g) * u) for the block's 8 intermediate
// columns.  XL: the activation rows are read from LDS (small batches),
// otherwise from global memory in the same pipeline as the weights.
// ----------------------------------------------------------------------------
template <int NMB, bool XL, int FMT>
struct GuStage {
  // tiles per stage (two stages are in flight)
  static constexpr int D = XL ? 4 : (NMB == 1 ? 2 : 1);
  typename WFmt<FMT>::W w[D];
  typename WFmt<FMT>::Scale s[D];
  u32x4 a[XL ? 1 : D][2][NMB];
};

template <int NMB, bool XL, int NMBMAX, int FMT>
__device__ __forceinline__ void gu_item(KParams& p, const Lds& L, int slot, int sbase, int r0, int nrows,
                        int rb, bool shared, int parity, int& pend) {
  flush_pending_now(L.ctr, pend);
  using Stage = GuStage<NMB, XL, FMT>;
  using Wt = typename WFmt<FMT>::W;
  using Sc = typename WFmt<FMT>::Scale;
  constexpr int D = Stage::D;
  const int w = wave_id(), lane = lane_id();
  const int n = lane & 15, kq = lane >> 4;
  const int nq = p.n_q13;
  const int nj = (nq - w + kWaves - 1) / kWaves;     // tiles of this wave
  const size_t blk = (size_t)slot * p.n_rb13 + rb;
  const Wt* wt = (const Wt*)p.w13p + blk * nq * kWave + lane;
  const Sc* sc = (const Sc*)p.s13p + blk * nq * kTileRows + n;

  // A operand rows: token of expert row r0 + mb*16 + n.  Rows past nrows read
  // row r0 (always valid) and are zeroed before the MFMA, so every load is
  // issued by every lane and the loads stay in order behind one counter.
  const uint16_t* arow[NMB];
  const SHARED uint16_t* arow_l[NMB];
  bool aval[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    const int r = mb * kMBlock + n;
    aval[mb] = r < nrows;
    const int rr = aval[mb] ? r : 0;
    const int tok = shared ? (r0 + rr) : (int)L.rows[sbase + r0 + rr];
    arow[mb] = p.x + (size_t)tok * p.H + 8 * kq;
    arow_l[mb] = L.xs + (size_t)tok * p.xs_stride + 8 * kq;
  }

  auto load = [&](Stage& S, int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int j = min(j0 + u, nj - 1);               // past the end: reload the last tile
      const int q = w + kWaves * j;
      S.w[u] = ld_stream(wt + (size_t)q * kWave);
      S.s[u] = ld_stream(sc + (size_t)q * kTileRows);
      if (!XL) {
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb)
            S.a[XL ? 0 : u][g][mb] = ld((const u32x4*)(arow[mb] + kTileK * q + kGroup * g));
      }
    }
  };
  f32x4 acc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) acc[mb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  auto compute = [&](const Stage& S, int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      if (j0 + u < nj) {
        const int q = w + kWaves * (j0 + u);
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const bf16x8 b = wdecode<FMT>(S.w[u], g);
          float s;
          if constexpr (FMT == kFmtFp8) s = g ? S.s[u].y : S.s[u].x;
          else s = mx_scale(S.s[u], g);
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) {
            u32x4 a;
            if (XL) a = *(const SHARED u32x4*)(arow_l[mb] + kTileK * q + kGroup * g);
            else a = S.a[XL ? 0 : u][g][mb];
            acc[mb] += s * mfma16(as_bf16x8(aval[mb] ? a : zero4), b);
          }
        }
      }
    }
  };
  // two register stages in turn; a stage is only loaded if it holds tiles
  // (the branches are uniform across the wave)
  Stage A, B;
  load(A, 0);
  for (int j0 = 0; j0 < nj; j0 += 2 * D) {
    if (j0 + D < nj) load(B, j0 + D);
    compute(A, j0);
    if (j0 + 2 * D < nj) load(A, j0 + 2 * D);
    if (j0 + D < nj) compute(B, j0 + D);
  }

  // cross-wave sum in fixed order (wave 0 + 1 + 2 + 3); the partials area
  // alternates between items, so the waves need no second barrier
  SHARED f32x4* red = (SHARED f32x4*)L.red + (parity & 1) * kWaves * NMBMAX * kWave;
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) red[(w * NMB + mb) * kWave + lane] = acc[mb];
  __syncthreads();
  // wave w finishes block w.  (Only the finishing waves store and count:
  // loads retire in order, so a wave that also stored here would wait for
  // those stores' acknowledgement before its next item's first MFMA.)
  if (w < NMB && w * kMBlock < nrows) {
    const int mb = w;
    f32x4 s = red[(0 * NMB + mb) * kWave + lane];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) s += red[(ww * NMB + mb) * kWave + lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) swiglu_out(p, L, s[i], i, sbase, r0 + mb * kMBlock, nrows - mb * kMBlock, rb);
    // each wave that stored h rows counts them in (one per 16-row block)
    if (lane == 0) count_done(L.ctr + kCtrHReady + slot * kLine);
  }
}

// ----------------------------------------------------------------------------
// Expert down projection: 128 output rows (8 row blocks, 2 per wave, full K =
// I) of one expert for up to 64 of its rows.  Output rows go to o_scr.  HL:
// the item's h rows (<= 16) are staged in LDS first; otherwise they are read
// from global memory in the weight pipeline.
// ----------------------------------------------------------------------------
template <int NMB, bool HL, int FMT>
struct DnStage {
  static constexpr int D = HL ? 4 : (NMB == 1 ? 2 : 1);
  typename WFmt<FMT>::W w[D][2];
  typename WFmt<FMT>::Scale s[D][2];
  u32x4 a[HL ? 1 : D][2][NMB];
};

template <int NMB, bool HL, int FMT>
__device__ __forceinline__ bool down_item(KParams& p, const Lds& L, int slot, int sbase, int r0, int nrows,
                          int rg, int h_target, int& pend) {
  flush_pending_now(L.ctr, pend);
  using Stage = DnStage<NMB, HL, FMT>;
  using Wt = typename WFmt<FMT>::W;
  using Sc = typename WFmt<FMT>::Scale;
  constexpr int D = Stage::D;
  const int w = wave_id(), lane = lane_id();
  const int n = lane & 15, kq = lane >> 4;
  const int nq = p.n_q2;
  const int rb0 = rg * (kDownRows / kTileRows) + 2 * w;
  const int nrb = min(2, p.n_rb2 - rb0);      // row blocks of this wave (0..2)

  const int nrb_eff = max(nrb, 1);            // waves past the last block idle after staging

  const uint64_t* arow[NMB];                  // tagged h words: 2 bf16 each
  const SHARED uint16_t* arow_l[NMB];
  bool aval[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    const int r = mb * kMBlock + n;
    aval[mb] = r < nrows;
    const int rr = aval[mb] ? r : 0;
    arow[mb] = p.h_scr + (size_t)(sbase + r0 + rr) * (p.I / 2) + 4 * kq;
    arow_l[mb] = L.hs + (size_t)rr * p.hs_stride + 8 * kq;
  }
  // a wave with a single row block (last group of a ragged H) loads that
  // block twice and stores only the first copy
  const Wt* wt[2];
  const Sc* sc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const size_t blk = (size_t)slot * p.n_rb2 + min(rb0 + min(j, nrb_eff - 1), p.n_rb2 - 1);
    wt[j] = (const Wt*)p.w2p + blk * nq * kWave + lane;
    sc[j] = (const Sc*)p.s2p + blk * nq * kTileRows + n;
  }
  auto load = [&](Stage& S, int q0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int q = min(q0 + u, nq - 1);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        S.w[u][j] = ld_stream(wt[j] + (size_t)q * kWave);
        S.s[u][j] = ld_stream(sc[j] + (size_t)q * kTileRows);
      }
      if (!HL) {
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb)
            S.a[HL ? 0 : u][g][mb] = ld_h8(arow[mb] + (kTileK * q + kGroup * g) / 2);
      }
    }
  };
  f32x4 acc[2][NMB];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) acc[j][mb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  auto compute = [&](const Stage& S, int q0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      if (q0 + u < nq) {
        const int q = q0 + u;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          u32x4 a[NMB];
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) {
            if (HL) a[mb] = *(const SHARED u32x4*)(arow_l[mb] + kTileK * q + kGroup * g);
            else a[mb] = S.a[HL ? 0 : u][g][mb];
            a[mb] = aval[mb] ? a[mb] : zero4;
          }
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const bf16x8 b = wdecode<FMT>(S.w[u][j], g);
            float s;
            if constexpr (FMT == kFmtFp8) s = g ? S.s[u][j].y : S.s[u][j].x;
            else s = mx_scale(S.s[u][j], g);
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) acc[j][mb] += s * mfma16(as_bf16x8(a[mb]), b);
          }
        }
      }
    }
  };
  Stage A, B;
  if (!HL) {
    // h is read in the pipeline below: it must be complete first
    if (!wait_geq(p, L.ctr + kCtrHReady + slot * kLine, h_target, L.misc + 1)) return false;
    if (!verify_h_rows(p, L, sbase + r0, nrows)) return false;
  }
  load(A, 0);                                 // weights first: they need no input
  if (HL) {
    // stage the item's h rows while the first weights are in flight (the
    // barrier inside the wait keeps the previous item's readers safe)
    if (!wait_geq(p, L.ctr + kCtrHReady + slot * kLine, h_target, L.misc + 1)) return false;
    if (!stage_h_rows(p, L, sbase + r0, nrows)) return false;
    __syncthreads();
  }
  if (nrb <= 0) return true;
  for (int q0 = 0; q0 < nq; q0 += 2 * D) {
    if (q0 + D < nq) load(B, q0 + D);
    compute(A, q0);
    if (q0 + 2 * D < nq) load(A, q0 + 2 * D);
    if (q0 + D < nq) compute(B, q0 + D);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (j < nrb) {
      const int rb = rb0 + j;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = mb * kMBlock + 4 * kq + i;
          if (r < nrows)
            st_tag(p.o_scr + (size_t)(sbase + r0 + r) * p.H + rb * kTileRows + n, __float_as_uint(acc[j][mb][i]), L.epoch);
        }
    }
  }
  pend = rg;
  return true;
}

// ----------------------------------------------------------------------------
// Fully unrolled gate/up and down items for the common shapes (x and h in LDS,
// one MFMA block): every weight tile of the wave's share is requested at the
// start of the item (16 KiB in flight per wave), then consumed in order, so
// each MFMA waits only for its own tile.
// ----------------------------------------------------------------------------
constexpr int kAhead = 2;                      // A operand tiles read ahead (full-tile items)

template <int NJ, int FMT>
__device__ __forceinline__ void gu_item_full(KParams& p, const Lds& L, int slot, int sbase, int r0, int nrows,
                             int rb, bool shared, int parity, int& pend) {
  using Wt = typename WFmt<FMT>::W;
  using Sc = typename WFmt<FMT>::Scale;
  const int w = wave_id(), lane = lane_id();
  const int n = lane & 15, kq = lane >> 4;
  const int nq = p.n_q13;                            // == 4 * NJ
  const size_t blk = (size_t)slot * p.n_rb13 + rb;
  const Wt* wt = (const Wt*)p.w13p + (blk * nq + w) * kWave + lane;
  const Sc* sc = (const Sc*)p.s13p + (blk * nq + w) * kTileRows + n;
  Wt wv[NJ];
  Sc sv[NJ];
  // issued in tile order (the scheduler may not reorder them: loads return
  // in issue order, so tile j must not wait for later tiles)
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    wv[j] = ld_stream(wt + (size_t)j * kWaves * kWave);
    sv[j] = ld_stream(sc + (size_t)j * kWaves * kTileRows);
    __builtin_amdgcn_sched_barrier(0);
  }
  flush_pending<2 * NJ>(L.ctr, pend);
  // Lanes past the item's rows read row 0: their products reach only output
  // rows that are never stored, so the operand needs no masking.
  const int nr = n < nrows ? n : 0;
  const int tok = shared ? r0 + nr : (int)L.rows[sbase + r0 + nr];
  const SHARED uint16_t* arow = L.xs + (size_t)tok * p.xs_stride + 8 * kq + kTileK * w;
  auto lda = [&](int j, int g) __attribute__((always_inline)) {
    return *(const SHARED u32x4*)(arow + kTileK * kWaves * j + kGroup * g);
  };
  // The A operands are read kAhead tiles ahead of their MFMAs, and each
  // MFMA's scaled sum is added one tile later, so neither the LDS nor the
  // MFMA latency stalls the wave; the sums keep the (tile, group) order.
  u32x4 a[NJ][2];
#pragma unroll
  for (int j = 0; j < kAhead && j < NJ; ++j) {
    a[j][0] = lda(j, 0);
    a[j][1] = lda(j, 1);
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (FMT == kFmtFp8) {
    f32x4 rl[2];
    float sl[2];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (j + kAhead < NJ) {
        a[j + kAhead][0] = lda(j + kAhead, 0);
        a[j + kAhead][1] = lda(j + kAhead, 1);
      }
      f32x4 r[2];
      float s[2];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        r[g] = mfma16(as_bf16x8(a[j][g]), wdecode<FMT>(wv[j], g));
        s[g] = g ? sv[j].y : sv[j].x;
      }
      if (j > 0) {
        acc += sl[0] * rl[0];
        acc += sl[1] * rl[1];
      }
      rl[0] = r[0];
      rl[1] = r[1];
      sl[0] = s[0];
      sl[1] = s[1];
    }
    acc += sl[0] * rl[0];
    acc += sl[1] * rl[1];
  } else {
    // MX: the scale goes into the decode; one running sum per group
    f32x4 ag[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (j + kAhead < NJ) {
        a[j + kAhead][0] = lda(j + kAhead, 0);
        a[j + kAhead][1] = lda(j + kAhead, 1);
      }
#pragma unroll
      for (int g = 0; g < 2; ++g)
        ag[g] = mfma16_acc(as_bf16x8(a[j][g]), wdecode_scaled<FMT>(wv[j], g, mx_scale(sv[j], g)), ag[g]);
    }
    acc = ag[0] + ag[1];
  }
  SHARED f32x4* red = (SHARED f32x4*)L.red + (parity & 1) * kWaves * kWave;
  red[w * kWave + lane] = acc;
  __syncthreads();
  // wave 0 finishes the block (see gu_item on why one wave)
  if (w == 0) {
    f32x4 s = red[lane];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) s += red[ww * kWave + lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) swiglu_out(p, L, s[i], i, sbase, r0, nrows, rb);
    if (lane == 0) count_done(L.ctr + kCtrHReady + slot * kLine);
  }
}

// The same for MXFP4 weights, two row blocks (2 rp, 2 rp + 1) per item: each
// wave has 2 NJ half-size tiles (16 KiB) in flight, as an FP8 item has, and
// every x operand read from LDS feeds both blocks' MFMAs.  Waves 0 and 1
// finish one block each.
template <int NJ>
__device__ __forceinline__ void gu_item_full_pair(KParams& p, const Lds& L, int slot, int sbase, int r0, int nrows,
                                                  int rp, bool shared, int parity, int& pend) {
  using Wt = typename WFmt<kFmtMxfp4>::W;
  using Sc = typename WFmt<kFmtMxfp4>::Scale;
  const int w = wave_id(), lane = lane_id();
  const int n = lane & 15, kq = lane >> 4;
  const int nq = p.n_q13;                            // == 4 * NJ
  Wt wv[2][NJ];
  Sc sv[2][NJ];
  const Wt* wt[2];
  const Sc* sc[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const size_t blk = (size_t)slot * p.n_rb13 + 2 * rp + b;
    wt[b] = (const Wt*)p.w13p + (blk * nq + w) * kWave + lane;
    sc[b] = (const Sc*)p.s13p + (blk * nq + w) * kTileRows + n;
  }
  // issued in the order the MFMAs consume them (K tile, then block), which
  // the scheduler may not change: loads return in issue order
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      wv[b][j] = ld_stream(wt[b] + (size_t)j * kWaves * kWave);
      sv[b][j] = ld_stream(sc[b] + (size_t)j * kWaves * kTileRows);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // 4 NJ = 64 loads are in flight; vmcnt holds at most 63, so the deferred
  // count also waits for the first of them (gate/up items rarely follow a
  // down item in this variant's list)
  flush_pending<(4 * NJ < 63 ? 4 * NJ : 63)>(L.ctr, pend);
  // lanes past the item's rows read row 0 (their output rows are not stored)
  const int nr = n < nrows ? n : 0;
  const int tok = shared ? r0 + nr : (int)L.rows[sbase + r0 + nr];
  const SHARED uint16_t* arow = L.xs + (size_t)tok * p.xs_stride + 8 * kq + kTileK * w;
  auto lda = [&](int j, int g) __attribute__((always_inline)) {
    return *(const SHARED u32x4*)(arow + kTileK * kWaves * j + kGroup * g);
  };
  // A read kAhead tiles ahead; each MFMA's scaled sum added one step later
  u32x4 a[NJ][2];
#pragma unroll
  for (int j = 0; j < kAhead && j < NJ; ++j) {
    a[j][0] = lda(j, 0);
    a[j][1] = lda(j, 1);
  }
  // the scale goes into the decode; one running sum per block and group
  f32x4 ag[2][2] = {{{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}, {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}};
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    if (j + kAhead < NJ) {
      a[j + kAhead][0] = lda(j + kAhead, 0);
      a[j + kAhead][1] = lda(j + kAhead, 1);
    }
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        ag[b][g] = mfma16_acc(as_bf16x8(a[j][g]), wdecode_scaled<kFmtMxfp4>(wv[b][j], g, mx_scale(sv[b][j], g)),
                              ag[b][g]);
  }
  f32x4 acc[2] = {ag[0][0] + ag[0][1], ag[1][0] + ag[1][1]};
  SHARED f32x4* red = (SHARED f32x4*)L.red + (parity & 1) * kWaves * 2 * kWave;
#pragma unroll
  for (int b = 0; b < 2; ++b) red[(b * kWaves + w) * kWave + lane] = acc[b];
  __syncthreads();
  if (w < 2) {
    const int b = w;
    f32x4 s = red[(b * kWaves + 0) * kWave + lane];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) s += red[(b * kWaves + ww) * kWave + lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) swiglu_out(p, L, s[i], i, sbase, r0, nrows, 2 * rp + b);
    if (lane == 0) count_done(L.ctr + kCtrHReady + slot * kLine);
  }
}

template <int NQ, int FMT>
__device__ __forceinline__ bool down_item_full(KParams& p, const Lds& L, int slot, int sbase, int r0, int nrows,
                               int rg, int h_target, int& pend) {
  using Wt = typename WFmt<FMT>::W;
  using Sc = typename WFmt<FMT>::Scale;
  const int w = wave_id(), lane = lane_id();
  const int n = lane & 15, kq = lane >> 4;
  const int rb0 = rg * (kDownRows / kTileRows) + 2 * w;
  const int nrb = min(2, p.n_rb2 - rb0);
  // The item's h rows (tagged words) are requested with its weights; when
  // every tag is current (h complete, the usual case) no counter needs to
  // be polled at all.
  constexpr int kHFast = 8;                   // h words per thread on the fast path
  const int per_row = p.I / 2;
  const int nh = nrows * per_row;
  const bool fast = nh <= kHFast * kThreads;
  const uint64_t* hsrc = p.h_scr + (size_t)(sbase + r0) * per_row;
  Wt wv[2][NQ];
  Sc sv[2][NQ];
  const Wt* wt[2];
  const Sc* sc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const size_t blk = (size_t)slot * p.n_rb2 + min(rb0 + j, p.n_rb2 - 1);
    wt[j] = (const Wt*)p.w2p + blk * NQ * kWave + lane;
    sc[j] = (const Sc*)p.s2p + blk * NQ * kTileRows + n;
  }
  auto ldw = [&](int q) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      wv[j][q] = ld_stream(wt[j] + (size_t)q * kWave);
      sv[j][q] = ld_stream(sc[j] + (size_t)q * kTileRows);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // Loads return in issue order, and the scheduler may not reorder these:
  // K tiles [0, NQ1) are requested before the h words and [NQ1, NQ) after
  // them, in the order the MFMAs consume them, so the first tiles' MFMAs
  // run while the last tiles arrive.
  constexpr int NQ1 = (NQ + 1) / 2;
#pragma unroll
  for (int q = 0; q < NQ1; ++q) ldw(q);
  uint64_t hv[kHFast];
  int nb = 0;
  if (fast) {
    // only the batches that hold words are issued (the condition is uniform)
#pragma unroll
    for (int b = 0; b < kHFast; ++b)
      hv[b] = b * kThreads < nh ? ld_tag(hsrc + min((int)threadIdx.x + b * kThreads, nh - 1)) : 0ull;
    nb = (nh + kThreads - 1) / kThreads;
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = NQ1; q < NQ; ++q) ldw(q);
  // the item's 4 NQ weight and scale loads and nb h loads are the youngest
  // operations: waiting for all but those covers the older stores
  flush_pending_rt<4 * NQ>(L.ctr, pend, nb);
  // the previous item's readers of the h area are done past this barrier
  __syncthreads();
  bool stale = !fast;
  if (fast) {
    // every word is written, to its place or (past the rows, or stale) to
    // the thread's scratch word, so the check has no per-word branches
    SHARED uint32_t* const sink = L.tks + threadIdx.x;
#pragma unroll
    for (int b = 0; b < kHFast; ++b) {
      const int i = threadIdx.x + b * kThreads;
      const bool ok = tag_ok(hv[b], L.epoch);
      const int r = (int)fdiv((uint32_t)i, p.fd_h2.m, p.fd_h2.s);
      SHARED uint32_t* const d = (SHARED uint32_t*)(L.hs + (size_t)r * p.hs_stride + 2 * (i - r * per_row));
      *(i < nh && ok ? d : sink) = (uint32_t)hv[b];
      stale |= i < nh && !ok;
    }
  }
  if (block_any(stale, L.misc + 8)) {
    // h not complete yet (or too many rows): wait for the count, then gather
    if (!wait_geq(p, L.ctr + kCtrHReady + slot * kLine, h_target, L.misc + 1)) return false;
    if (!stage_h_rows(p, L, sbase + r0, nrows)) return false;
  } else if (threadIdx.x == 0) {
    *(SHARED long long*)(L.misc + 12) = tl_clock(p);   // inputs ready (timeline)
  }
  __syncthreads();
  if (nrb <= 0) return true;
  // lanes past the item's rows read row 0 (their output rows are not stored)
  const SHARED uint16_t* arow = L.hs + (size_t)(n < nrows ? n : 0) * p.hs_stride + 8 * kq;
  // (K tile, group) steps st = 2 q + g: A read 2 kAhead steps ahead, each
  // MFMA's scaled sum added one step later, in the same order
  constexpr int NS = 2 * NQ;
  u32x4 a[NS];
#pragma unroll
  for (int st = 0; st < 2 * kAhead && st < NS; ++st) a[st] = *(const SHARED u32x4*)(arow + kGroup * st);
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  if constexpr (FMT == kFmtFp8) {
    f32x4 rl[2];
    float sl[2];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      if (st + 2 * kAhead < NS) a[st + 2 * kAhead] = *(const SHARED u32x4*)(arow + kGroup * (st + 2 * kAhead));
      const int q = st >> 1, g = st & 1;
      f32x4 r[2];
      float s[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        r[j] = mfma16(as_bf16x8(a[st]), wdecode<FMT>(wv[j][q], g));
        s[j] = g ? sv[j][q].y : sv[j][q].x;
      }
      if (st > 0) {
        acc[0] += sl[0] * rl[0];
        acc[1] += sl[1] * rl[1];
      }
      rl[0] = r[0];
      rl[1] = r[1];
      sl[0] = s[0];
      sl[1] = s[1];
    }
    acc[0] += sl[0] * rl[0];
    acc[1] += sl[1] * rl[1];
  } else {
    // MX: the scale goes into the decode; one running sum per block and group
    f32x4 ag[2][2] = {{{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}, {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}};
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      if (st + 2 * kAhead < NS) a[st + 2 * kAhead] = *(const SHARED u32x4*)(arow + kGroup * (st + 2 * kAhead));
      const int q = st >> 1, g = st & 1;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        ag[j][g] = mfma16_acc(as_bf16x8(a[st]), wdecode_scaled<FMT>(wv[j][q], g, mx_scale(sv[j][q], g)), ag[j][g]);
    }
    acc[0] = ag[0][0] + ag[0][1];
    acc[1] = ag[1][0] + ag[1][1];
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (j < nrb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * kq + i;
        if (r < nrows)
          st_tag(p.o_scr + (size_t)(sbase + r0 + r) * p.H + (rb0 + j) * kTileRows + n, __float_as_uint(acc[j][i]), L.epoch);
      }
    }
  }
  pend = rg;
  return true;
}

// ----------------------------------------------------------------------------
// Wide items: batches above 16 rows at H = 64 kWideTiles and I = 512, 576 or 640,
// up to kWideRows (two MFMA blocks) rows of one expert per item, two
// workgroups per compute unit.
//
// Gate/up: kWideRb row blocks (4 x 16 weight rows, 256 KiB of FP8) of one
// expert.  Wave w takes K tiles [16 w, 16 w + 16) of all four blocks, so every
// activation value it loads (from global memory; the batch does not fit in
// LDS) feeds four blocks' MFMAs; four K steps (16 weight tiles) are in flight
// per wave.  The waves' partial sums meet in LDS and wave w finishes block
// kWideRb rg + w, summing the four K quarters in wave order.
// ----------------------------------------------------------------------------
template <int NMB, int FMT>
__device__ __forceinline__ void gu_item_wide(KParams& p, const Lds& L, int slot, int sbase, int r0, int nrows,
                                             int rg, bool shared, int& pend) {
  using Wt = typename WFmt<FMT>::W;
  using Sc = typename WFmt<FMT>::Scale;
  constexpr int NJ = kWideTiles;               // K tiles per wave
  constexpr int P = NMB == 1 ? 4 : 3;          // K steps in flight
  const int w = wave_id(), lane = lane_id();
  const int n = lane & 15, kq = lane >> 4;
  const int nq = p.n_q13;
  const int q0 = NJ * w;
  const Wt* wt[kWideRb];
  const Sc* sc[kWideRb];
#pragma unroll
  for (int r = 0; r < kWideRb; ++r) {
    const size_t blk = (size_t)slot * p.n_rb13 + kWideRb * rg + r;
    wt[r] = (const Wt*)p.w13p + (blk * nq + q0) * kWave + lane;
    sc[r] = (const Sc*)p.s13p + (blk * nq + q0) * kTileRows + n;
  }
  // A operand rows: rows past nrows read row r0.  Their products reach only
  // output rows that are never stored, so zeroing them is not needed; it is
  // kept for the byte formats, whose loops measured faster with it, and
  // dropped for MXFP4, whose loop (half the bytes per MFMA) pays for the
  // selects' issue slots
  const uint16_t* arow[NMB];
  bool aval[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    const int r = mb * kMBlock + n;
    aval[mb] = r < nrows;
    const int rr = aval[mb] ? r : 0;
    const int tok = shared ? (r0 + rr) : (int)L.rows[sbase + r0 + rr];
    arow[mb] = p.x + (size_t)tok * p.H + kTileK * q0 + 8 * kq;
  }
  struct Step {
    u32x4 a[2][NMB];
    Wt w[kWideRb];
    Sc s[kWideRb];
  };
  Step S[P];
  auto load = [&](Step& st_, int j) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) st_.a[g][mb] = ld((const u32x4*)(arow[mb] + kTileK * j + kGroup * g));
#pragma unroll
    for (int r = 0; r < kWideRb; ++r) {
      st_.w[r] = ld_stream(wt[r] + (size_t)j * kWave);
      st_.s[r] = ld_stream(sc[r] + (size_t)j * kTileRows);
    }
  };
#pragma unroll
  for (int j = 0; j < P; ++j) load(S[j], j);
  flush_pending<P * (2 * NMB + 2 * kWideRb)>(L.ctr, pend);
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  f32x4 acc[kWideRb][NMB];
#pragma unroll
  for (int r = 0; r < kWideRb; ++r)
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) acc[r][mb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // step j lives in S[j % P]; the inner loop keeps that index a constant
#pragma unroll
  for (int j0 = 0; j0 < NJ; j0 += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int j = j0 + u;
      if (j < NJ) {
        Step& st_ = S[u];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          bf16x8 a[NMB];
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb)
            a[mb] = as_bf16x8(FMT == kFmtMxfp4 || aval[mb] ? st_.a[g][mb] : zero4);
#pragma unroll
          for (int r = 0; r < kWideRb; ++r) {
            if constexpr (FMT == kFmtFp8) {
              const bf16x8 b = fp8x8_to_bf16(st_.w[r][2 * g], st_.w[r][2 * g + 1]);
              const float s = g ? st_.s[r].y : st_.s[r].x;
#pragma unroll
              for (int mb = 0; mb < NMB; ++mb) acc[r][mb] += s * mfma16(a[mb], b);
            } else {
              // MX: the scale goes into the decode (exact), the MFMA accumulates
              const bf16x8 b = wdecode_scaled<FMT>(st_.w[r], g, mx_scale(st_.s[r], g));
#pragma unroll
              for (int mb = 0; mb < NMB; ++mb) acc[r][mb] = mfma16_acc(a[mb], b, acc[r][mb]);
            }
          }
        }
        // pin the sums here, step by step, so the step's registers are free
        // for its reload (else the compiler reorders the ring and waits on
        // loads it has only just issued)
#pragma unroll
        for (int r = 0; r < kWideRb; ++r)
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) asm volatile("" : "+v"(acc[r][mb]));
        if (j + P < NJ) load(st_, j + P);
      }
    }
  }
  // the first barrier also ends the previous item's reads of the area
  __syncthreads();
  SHARED f32x4* red = (SHARED f32x4*)L.red;    // [kWaves][kWideRb][NMB][64]
#pragma unroll
  for (int r = 0; r < kWideRb; ++r)
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) red[((w * kWideRb + r) * NMB + mb) * kWave + lane] = acc[r][mb];
  __syncthreads();
  const int rb = kWideRb * rg + w;
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    if (mb * kMBlock < nrows) {
      f32x4 s = red[((0 * kWideRb + w) * NMB + mb) * kWave + lane];
#pragma unroll
      for (int ww = 1; ww < kWaves; ++ww) s += red[((ww * kWideRb + w) * NMB + mb) * kWave + lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) swiglu_out(p, L, s[i], i, sbase, r0 + mb * kMBlock, nrows - mb * kMBlock, rb);
    }
  }
  // one publication per wave and item: an M-range counts n_rb13 in all
  if (lane == 0) count_done(L.ctr + kCtrHReady + slot * kLine);
}

// ----------------------------------------------------------------------------
// Wide down item: 512 output rows of one expert (wave w: the 128-row column
// group 4 rg + w, kWideDnBlocks row blocks) for up to kWideRows rows.  The
// wave's first 16 weight tiles are requested before the item waits for its
// expert's gate/up items; then the item's h rows go to LDS and the wave runs
// K tile by K tile, each h operand feeding its 8 row blocks, 16 tiles in
// flight.
// ----------------------------------------------------------------------------
template <int NMB, int NQ, int FMT>
__device__ __forceinline__ bool dn_item_wide(KParams& p, const Lds& L, int slot, int sbase, int r0, int nrows,
                                             int rg, int h_target, int& pend) {
  using Wt = typename WFmt<FMT>::W;
  using Sc = typename WFmt<FMT>::Scale;
  constexpr int NB = kWideDnBlocks;
  constexpr int NT = NB * NQ;                  // NQ K tiles per row block: I = 64 NQ
  constexpr int P = NMB == 1 ? 16 : 8;         // tiles in flight
  const int w = wave_id(), lane = lane_id();
  const int n = lane & 15, kq = lane >> 4;
  const int grp = rg * kWaves + w;             // this wave's 128-column group
  const size_t blk0 = (size_t)slot * p.n_rb2 + (size_t)grp * NB;
  const Wt* wt = (const Wt*)p.w2p + blk0 * NQ * kWave + lane;
  const Sc* sc = (const Sc*)p.s2p + blk0 * NQ * kTileRows + n;
  // tile t = NB q + b is K tile q of row block b; the ring turns over P / NB
  // K steps at a time (the last turn may hold fewer when P does not divide NT)
  static_assert(P % NB == 0 && NT >= P, "tile ring");
  Wt wv[P];
  Sc sv[P];
  // tile t into ring slot u = t mod P (u passed as a constant)
  auto load = [&](int t, int u) __attribute__((always_inline)) {
    const int q = t / NB, b = t % NB;
    wv[u] = ld_stream(wt + (size_t)(b * NQ + q) * kWave);
    sv[u] = ld_stream(sc + (size_t)(b * NQ + q) * kTileRows);
  };
#pragma unroll
  for (int t = 0; t < P; ++t) load(t, t);
  flush_pending<2 * P>(L.ctr, pend);
  // the barriers of the wait also end the previous item's reads of the area
  if (!wait_geq(p, L.ctr + kCtrHReady + slot * kLine, h_target, L.misc + 1)) return false;
  if (!stage_h_rows(p, L, sbase + r0, nrows)) return false;
  __syncthreads();
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  const SHARED uint16_t* arow[NMB];
  bool aval[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    const int r = mb * kMBlock + n;
    aval[mb] = r < nrows;
    arow[mb] = L.hs + (size_t)(aval[mb] ? r : 0) * p.hs_stride + 8 * kq;
  }
  f32x4 acc[NB][NMB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) acc[b][mb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t0 = 0; t0 < NT; t0 += P) {
#pragma unroll
    for (int qq = 0; qq < P / NB; ++qq) {
      const int q = t0 / NB + qq;
      if (q >= NQ) continue;                   // resolved at compile time
      bf16x8 a[2][NMB];
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
          a[g][mb] = as_bf16x8(FMT == kFmtMxfp4 || aval[mb] ? *(const SHARED u32x4*)(arow[mb] + kTileK * q + kGroup * g)
                                                             : zero4);   // (rows past nrows: as in gu_item_wide)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int u = qq * NB + b;             // ring slot of tile t0 + u
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          if constexpr (FMT == kFmtFp8) {
            const bf16x8 bw = fp8x8_to_bf16(wv[u][2 * g], wv[u][2 * g + 1]);
            const float s = g ? sv[u].y : sv[u].x;
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) acc[b][mb] += s * mfma16(a[g][mb], bw);
          } else {
            // MX: the scale goes into the decode (exact), the MFMA accumulates
            const bf16x8 bw = wdecode_scaled<FMT>(wv[u], g, mx_scale(sv[u], g));
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) acc[b][mb] = mfma16_acc(a[g][mb], bw, acc[b][mb]);
          }
        }
        // pin the sums here, in tile order (else the compiler runs every MFMA
        // first and keeps all their results for the multiply-adds at the end)
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) asm volatile("" : "+v"(acc[b][mb]));
        if (t0 + u + P < NT) load(t0 + u + P, u);
      }
    }
  }
  // the sums are final here: without this the compiler sinks each element's
  // whole multiply-add chain into its conditional store below, which keeps
  // every MFMA result alive to the end of the item
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) asm volatile("" : "+v"(acc[b][mb]));
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mb * kMBlock + 4 * kq + i;
        if (r < nrows)
          st_tag(p.o_scr + (size_t)(sbase + r0 + r) * p.H + (grp * NB + b) * kTileRows + n,
                 __float_as_uint(acc[b][mb][i]), L.epoch);
      }
  pend = grp;
  return true;
}

// ----------------------------------------------------------------------------
// Pre-norm block runs: the input RMSNorm in the kernel's prologue, rows handed
// on one by one as they become ready.  Workgroup G - 1 - g normalises rows g,
// g + G, ...: xn[t][h] = bf16(x[t][h] r_t gamma[h]), r_t = 1 / sqrt(mean_h x[t][h]^2
// + eps), the mean in fp32 in a fixed order.  The row goes out with
// device-scope stores (to the device coherence point, past this XCD's L2);
// once every wave's stores are acknowledged, thread 0 sets the row's ready
// word to the run's epoch.  A reader waits for the words of the rows it needs
// and then reads them with ordinary loads: no L1 or L2 can hold a stale line
// of a row, since nothing reads it in this run before its word is set and the
// caches start each kernel clean.  The prologue comes before any wait, so the
// rows are ready while all workgroups are resident.
// ----------------------------------------------------------------------------
constexpr int kNormChunks = 16384 / 8 / kThreads;   // 16-byte words per thread at the largest H
__device__ __forceinline__ void st_coh64(uint64_t* p, uint64_t v) {
  __hip_atomic_store((GLOBAL uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void norm_rows(KParams& p, const Lds& L) {
  SHARED float* const red = L.red;
  const int n8 = p.H / 8;
  // the last workgroups take the rows: the first ones start the router items,
  // which wait for every row anyway
  for (int t = gridDim.x - 1 - blockIdx.x; t < p.T; t += gridDim.x) {
    const u32x4* src = (const u32x4*)(p.x_in + (size_t)t * p.H);
    const f32x4* gw = (const f32x4*)p.norm_w;
    u32x4 v[kNormChunks];
    f32x4 g[kNormChunks][2];
#pragma unroll
    for (int j = 0; j < kNormChunks; ++j) {
      const int c = (int)threadIdx.x + j * kThreads;
      if (c < n8) {
        v[j] = ld(src + c);
        g[j][0] = ld(gw + 2 * c);
        g[j][1] = ld(gw + 2 * c + 1);
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < kNormChunks; ++j) {
      if ((int)threadIdx.x + j * kThreads < n8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = bf16_to_f32(v[j][i] & 0xffffu), b = bf16_to_f32(v[j][i] >> 16);
          ss = fmaf(a, a, ss);
          ss = fmaf(b, b, ss);
        }
      }
    }
    ss = wave_sum(ss);
    if (lane_id() == 0) red[wave_id()] = ss;
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();                           // the partials area is free again
    const float r = 1.0f / sqrtf(tot / (float)p.H + p.norm_eps);
    uint64_t* dst = (uint64_t*)(p.xn + (size_t)t * p.H);
#pragma unroll
    for (int j = 0; j < kNormChunks; ++j) {
      const int c = (int)threadIdx.x + j * kThreads;
      if (c < n8) {
        const float gg[8] = {g[j][0].x, g[j][0].y, g[j][0].z, g[j][0].w, g[j][1].x, g[j][1].y, g[j][1].z, g[j][1].w};
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t lo = f32_to_bf16(bf16_to_f32(v[j][i] & 0xffffu) * r * gg[2 * i]);
          const uint32_t hi = f32_to_bf16(bf16_to_f32(v[j][i] >> 16) * r * gg[2 * i + 1]);
          o[i] = lo | hi << 16;
        }
        st_coh64(dst + 2 * c, (uint64_t)o.y << 32 | o.x);
        st_coh64(dst + 2 * c + 1, (uint64_t)o.w << 32 | o.z);
        if (p.dbg_norm) st((u32x4*)(p.dbg_norm + (size_t)t * p.H) + c, o);
      }
    }
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0) store_agent(p.norm_ready + t, (int)L.epoch);
  }
}

// Workgroup-wide wait until rows [t0, t0 + n) of xn are ready: the lanes of
// wave 0 poll one ready word each, under the deadline.  false: deadline
// passed or another workgroup reported an error.
__device__ bool wait_rows(KParams& p, const Lds& L, int t0, int n) {
  SHARED int* const lds_flag = L.misc + 1;
  if ((int)threadIdx.x < kWave) {
    uint32_t bad = 0;
    long long t_end = 0;
    bool timed = false;
    for (int r = threadIdx.x; r < n && !bad; r += kWave) {
      int spins = 0;
      while (load_agent(p.norm_ready + t0 + r) != (int)L.epoch) {
        if (!timed) {
          t_end = (long long)wall_clock64() + (p.expire_waits ? 0 : p.deadline_ticks);
          timed = true;
        }
        if ((spins & 7) == 7 && load_agent(p.status) != 0) { bad = 1; break; }
        if ((long long)wall_clock64() > t_end) {
          int expected = 0;
          __hip_atomic_compare_exchange_strong((GLOBAL int*)(p.status), &expected, MOE_ERR_TIMEOUT,
                                               __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
          bad = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
        ++spins;
      }
    }
    bad = wave_max_v(bad);
    if (threadIdx.x == 0) *lds_flag = bad ? 0 : 1;
  }
  __syncthreads();
  const int ok = *lds_flag;
  __syncthreads();
  return ok != 0;
}

// ----------------------------------------------------------------------------
// The persistent kernel
// ----------------------------------------------------------------------------
// FULL: the variant for x in LDS with the full-tile gate/up and down items
// (H = 64 kFullTiles, I = 32 kFullTiles or, NQ2 = kFullTiles / 2 + 1, 576)
// and local routing only; the other variants hold the general code.  Each variant
// carries only the code its batches reach, which keeps register pressure
// (and spills) down.  FMT: the expert weight format (WFmt).
template <int NMBMAX, bool XL, bool FULL, bool WIDE, int NQ2 = kFullTiles / 2, bool NORM = false, int FMT = kFmtFp8,
          bool PAIR = false>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(NMBMAX == 1 || WIDE ? 2 : 1))) moe_decode_kernel(Params arg) {
  static_assert(!PAIR || (FULL && FMT == kFmtMxfp4), "paired gate/up items: full-tile MXFP4 only");
  KParams& p = *(const CONSTANT Params*)__builtin_amdgcn_kernarg_segment_ptr();
  (void)arg;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  Lds L = lds_view(p, (SHARED char*)smem);
  const int tid = threadIdx.x;
  const int G = gridDim.x;
  // Small batch: the whole layer input is kept in LDS, loaded before the
  // first item that reads it (the router reads x from global memory, so the
  // copy overlaps the routing wait).
  // NORM: x is xn, whose rows are written by the prologue (every read of
  // it waits for the rows it needs first).
  bool x_staged = !XL;
  bool rows_all = !NORM;        // every xn row seen ready by this workgroup
  auto ensure_x = [&]() __attribute__((always_inline)) -> bool {
    if (x_staged) return true;
    if constexpr (NORM) {
      if (!wait_rows(p, L, 0, p.T)) return false;
      rows_all = true;
    }
    const int per_row = p.H / 8;
    batched_copy<u32x4>(
        p.T * per_row, [&](int i) { return ld((const u32x4*)p.x + i); },
        [&](int i, u32x4 v) {
          const int r = (int)fdiv((uint32_t)i, p.fd_x8.m, p.fd_x8.s);
          *(SHARED u32x4*)(L.xs + (size_t)r * p.xs_stride + 8 * (i - r * per_row)) = v;
        });
    __syncthreads();
    x_staged = true;
    return true;
  };
  bool routed = false;          // routing and placement are in LDS
  int i_rgu_end = 0, i_sdn_end = 0, i_rdn_end = 0, i_total = 0, n_mr = 0;

  // Arrival: this run's index, hence its tag and counter block (see
  // kArriveGroups).  Every workgroup arrives before anything else, so the
  // counters advance by exactly kRunUnits per run even when a wait fails.
  // Thread 0 requests it at once; the answer is read (arrival_take, thread
  // 0, then a barrier, then arrival_use) right away, except in a workgroup
  // whose first item is a small-batch router item: that item issues its
  // loads first and takes the answer at its partial-sum barrier, since it
  // needs the tag only for its stores.
  unsigned long long arrival = 0;
  if (tid == 0) {
    const int cg = (int)blockIdx.x % kArriveGroups;
    const int in_group = (G - 1 - cg) / kArriveGroups + 1;
    const unsigned long long add = (int)blockIdx.x < kArriveGroups ? kRunUnits - (unsigned)(in_group - 1) : 1ull;
    arrival = __hip_atomic_fetch_add((GLOBAL unsigned long long*)(p.arrive + cg * (kLine / 2)), add,
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  auto arrival_take = [&]() __attribute__((always_inline)) {
    if (tid == 0) {
      const unsigned long long n = arrival >> kRunUnitsLog2;
      s_run.epoch = (uint32_t)(n % 0xffffffffull) + 1u;
      s_run.ctr = p.ctr_base + (size_t)(n & 1) * kCtrHead;
    }
  };
  auto arrival_use = [&]() __attribute__((always_inline)) {
    L.epoch = __builtin_amdgcn_readfirstlane(s_run.epoch);
    const uint64_t a = (uint64_t)s_run.ctr;
    L.ctr = (int*)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                   (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a));
    // The last workgroup clears the other counter block for the next run (no
    // one uses it during this run): every counter any shape can use.
    if ((int)blockIdx.x == G - 1) {
      int* q = p.ctr_base + (L.ctr == p.ctr_base ? kCtrHead : 0);
      constexpr int n_words = 1 + kClaimGroups + (kMaxExperts + 1) + kMaxRowGroups + kGoLines;
      for (int i = tid; i < n_words; i += kThreads) {
        int off;
        if (i < 1) off = kCtrTopkDone;
        else if (i < 1 + kClaimGroups) off = kCtrTicket + (i - 1) * kLine;
        else if (i < 1 + kClaimGroups + kMaxExperts + 1) off = kCtrHReady + (i - 1 - kClaimGroups) * kLine;
        else if (i < 1 + kClaimGroups + kMaxExperts + 1 + kMaxRowGroups)
          off = kCtrRgDone + (i - 1 - kClaimGroups - kMaxExperts - 1) * kLine;
        else off = kCtrTopkGo + (i - 1 - kClaimGroups - kMaxExperts - 1 - kMaxRowGroups) * kGoStride;
        store_agent(q + off, 0);
      }
    }
  };
  // (full-tile kernels: the router item is the workgroup's first item, run
  // before the item loop below, so the answer is not held across the loop)
  const bool arrival_lazy = FULL && !NORM && (int)blockIdx.x < p.i_router_end;
  if (!arrival_lazy) {
    arrival_take();
    __syncthreads();
    arrival_use();
  }

  if constexpr (NORM) norm_rows(p, L);

  // optional timeline of this workgroup (thread 0 writes it)
  long long* trace = (p.trace && (int)blockIdx.x < p.trace_blocks)
                         ? p.trace + (size_t)blockIdx.x * (1 + p.trace_cap) * 4 : nullptr;
  const long long t_entry = tl_clock(p);
  int n_ev = 0;
  long long t_got = 0, t_ready = 0;
  int kind = 0, it = 0;
  auto record = [&]() __attribute__((always_inline)) {
    if (trace && tid == 0 && n_ev < p.trace_cap) {
      long long* r = trace + (size_t)(1 + n_ev) * 4;
      st(r + 0, (long long)it | ((long long)kind << 32));
      st(r + 1, t_got);
      st(r + 2, t_ready);
      st(r + 3, (long long)wall_clock64());
    }
    ++n_ev;
  };

  // Routing in this workgroup: top-k (selected here for small batches, else
  // copied from the distributed top-k items) and the bitmap placement.
  auto ensure_routing = [&]() __attribute__((always_inline)) -> bool {
    if (routed) return true;
    const long long r_start = tl_clock(p);
    if constexpr (WIDE) __syncthreads();       // the bitmaps share an area with earlier items' partial sums
    clear_placement(p, L);                     // the barriers of the waits below order it
    long long r_go = 0, r_lg = 0, r_row0 = 0, c_lg = 0;
    uint32_t touch = 0;
    if (FULL && (int)blockIdx.x >= p.i_pre_end) touch = touch_weight_pages(p, (int)blockIdx.x - p.i_pre_end, G - p.i_pre_end);
    if (FULL || p.local_topk) {
      // all T x E logits into LDS: the router items' tagged words are
      // polled directly (no completion count), late ones round by round
      __syncthreads();                         // earlier readers of the lg area are done
      r_go = tl_clock(p);
      if (!gather_logits(p, L)) return false;
      __syncthreads();
      r_lg = tl_clock(p);
      c_lg = tl_cycles(p);
      // rows 2w, 2w+1 (then 2w+8, 2w+9): one pair per wave, a row per half
      for (int t0 = 2 * wave_id(); t0 < p.T; t0 += 2 * kWaves) {
        const int t1 = min(t0 + 1, p.T - 1);
        int e;
        float wk;
        topk_pair(p, L.lg, t0, t1, &e, &wk);
        if (t0 == 0) r_row0 = tl_clock(p);
        const int hl = lane_id() & 31;
        const int t = lane_id() < 32 ? t0 : t0 + 1;
        if (hl < p.K && t < p.T) {
          L.tki[t * p.K + hl] = (int16_t)e;
          L.tkw[t * p.K + hl] = wk;
        }
      }
      if (touch == 0x9e3779b9u) L.misc[15] = 1;   // keeps the page touches alive
    } else if constexpr (!FULL) {
      if (!wait_geq(p, go_flag(L.ctr + kCtrTopkGo), 1, L.misc + 1, 1 << 20)) return false;
      // indices, then weights, kBatch loads in flight per thread
      const int tk = p.T * p.K;
      batched_copy<int>(
          2 * tk, [&](int i) { return i < tk ? ld_coh(p.topk_idx + i) : __float_as_int(ld_coh(p.topk_w + i - tk)); },
          [&](int i, int v) {
            if (i < tk) L.tki[i] = (int16_t)v;
            else L.tkw[i - tk] = __int_as_float(v);
          });
    }
    const long long r_rows = tl_clock(p);
    const long long c_rows = tl_cycles(p);
    __syncthreads();
    const long long r_topk = tl_clock(p);
    build_placement(p, L);
    const long long r_place = tl_clock(p);
    if (blockIdx.x == 0) write_routing_debug(p, L);
    if (trace && tid == 0 && n_ev + 1 < p.trace_cap) {   // routing phases: kinds 8, 9
      long long* r = trace + (size_t)(1 + n_ev) * 4;
      st(r + 0, (long long)8 << 32 | (long long)((r_place - r_topk) & 0xffffffff));
      st(r + 1, r_start);
      st(r + 2, r_go);
      st(r + 3, r_topk);
      r += 4;
      st(r + 0, (long long)9 << 32 | (long long)((c_rows - c_lg) & 0xffff) | (long long)min(L.misc[14], 0xffff) << 16);
      st(r + 1, r_lg);
      st(r + 2, r_row0);
      st(r + 3, r_rows);
      n_ev += 2;
      if (n_ev < p.trace_cap) {                // kind 10: ends of the logits gather's first rounds
        r += 4;
        st(r + 0, (long long)10 << 32);
        for (int i = 0; i < 3; ++i) st(r + 1 + i, i <= L.misc[14] ? ((SHARED long long*)(L.misc + 16))[i] : 0ll);
        ++n_ev;
      }
    }
    n_mr = L.misc[0];
    i_rgu_end = p.i_pre_end + n_mr * p.n_gu_mr;
    i_sdn_end = i_rgu_end + p.n_sdn;
    i_rdn_end = i_sdn_end + n_mr * p.n_dn_mr;
    i_total = i_rdn_end + p.n_cmb;
    routed = true;
    return true;
  };

  int gu_count = 0;             // parity of the gate/up partial-sum area
  int pend_rg = -1;             // this wave's deferred column-group count (-1: none)
  auto run_gu = [&](int slot, int sbase, int r0, int nrows, int rb, bool shared) __attribute__((always_inline)) {
    const int nmb = (nrows + kMBlock - 1) / kMBlock;
    const int par = gu_count++;
    if constexpr (WIDE) {
      if (nmb <= 1) gu_item_wide<1, FMT>(p, L, slot, sbase, r0, nrows, rb, shared, pend_rg);
      else gu_item_wide<2, FMT>(p, L, slot, sbase, r0, nrows, rb, shared, pend_rg);
    } else if constexpr (PAIR) {
      // launched only for lists built for pairs (gu_pair: n_gu_mr = n_rb13 / 2,
      // rb the pair index; checked on the host)
      gu_item_full_pair<kFullTiles>(p, L, slot, sbase, r0, nrows, rb, shared, par, pend_rg);
    } else if constexpr (FULL) gu_item_full<kFullTiles, FMT>(p, L, slot, sbase, r0, nrows, rb, shared, par, pend_rg);
    else if (NMBMAX == 1 || nmb <= 1) gu_item<1, XL, NMBMAX, FMT>(p, L, slot, sbase, r0, nrows, rb, shared, par, pend_rg);
    else if (nmb == 2) gu_item<NMBMAX >= 2 ? 2 : 1, XL, NMBMAX, FMT>(p, L, slot, sbase, r0, nrows, rb, shared, par, pend_rg);
    else if (nmb == 3) gu_item<NMBMAX >= 3 ? 3 : 1, XL, NMBMAX, FMT>(p, L, slot, sbase, r0, nrows, rb, shared, par, pend_rg);
    else gu_item<NMBMAX >= 4 ? 4 : 1, XL, NMBMAX, FMT>(p, L, slot, sbase, r0, nrows, rb, shared, par, pend_rg);
  };
  // a down item waits (after issuing its first weight loads) until its
  // expert's gate/up items have counted in ht publications
  auto run_down = [&](int slot, int sbase, int r0, int nrows, int rg, int ht) __attribute__((always_inline)) -> bool {
    const int nmb = (nrows + kMBlock - 1) / kMBlock;
    if constexpr (WIDE) {
      if (nmb <= 1) return dn_item_wide<1, NQ2, FMT>(p, L, slot, sbase, r0, nrows, rg, ht, pend_rg);
      return dn_item_wide<2, NQ2, FMT>(p, L, slot, sbase, r0, nrows, rg, ht, pend_rg);
    } else if constexpr (FULL) return down_item_full<NQ2, FMT>(p, L, slot, sbase, r0, nrows, rg, ht, pend_rg);
    else if (XL && p.hs_stride > 0) return down_item<1, XL, FMT>(p, L, slot, sbase, r0, nrows, rg, ht, pend_rg);
    else if (NMBMAX == 1 || nmb <= 1) return down_item<1, false, FMT>(p, L, slot, sbase, r0, nrows, rg, ht, pend_rg);
    else if (nmb == 2) return down_item<NMBMAX >= 2 ? 2 : 1, false, FMT>(p, L, slot, sbase, r0, nrows, rg, ht, pend_rg);
    else if (nmb == 3) return down_item<NMBMAX >= 3 ? 3 : 1, false, FMT>(p, L, slot, sbase, r0, nrows, rg, ht, pend_rg);
    else return down_item<NMBMAX >= 4 ? 4 : 1, false, FMT>(p, L, slot, sbase, r0, nrows, rg, ht, pend_rg);
  };
  // gate/up publications an expert's down items wait for: per gate/up row
  // block, one per 16-row MFMA block (wide items: one per 32-row M-range)
  auto h_target = [&](int rows) __attribute__((always_inline)) {
    return p.n_rb13 * ((rows + p.h_rows_per_count - 1) / p.h_rows_per_count);
  };

  // Schedule.  Items [0, S) are static: workgroup g takes g, g + G, ... in
  // order.  The items [S, i_total) are claimed, S = the later of the end of
  // the gate/up items and i_total - G, so the tail balances itself: claim group c = g mod 8 owns items S + c, S + c + 8, ...
  // and hands them out in order from its own counter (eight counters on
  // separate lines, so simultaneous claims do not queue on one address).  A
  // claim is issued when an item starts and read when it ends, so its round
  // trip hides behind the item.  An item waits only on items earlier in the
  // list, each workgroup's items increase, a group's claims come in order
  // and a workgroup claims only after its static items: the earliest
  // unfinished item is always being worked on, so every wait ends while all
  // workgroups are resident.  S needs the routing (i_total).
  bool dyn = false;
  int i_dyn = INT_MAX;          // S, once routed
  const int cgroup = blockIdx.x % kClaimGroups;
  auto claim_ctr = [&]() __attribute__((always_inline)) { return L.ctr + kCtrTicket + cgroup * kLine; };
  it = blockIdx.x;
  if (arrival_lazy) {
    // the first item, a router item, which also reads the run's arrival
    kind = 0;
    t_got = t_ready = tl_clock(p);
    const bool stage = !x_staged && p.T <= kRouterRows;
    t_ready = router_item<NORM>(p, L, it, stage, arrival_take, arrival_use);
    x_staged = x_staged || stage;
    record();
    it += G;
  }
  for (;;) {
    if (!dyn && it >= p.i_pre_end) {
      if (!ensure_x()) break;
      if (!ensure_routing()) break;
      // Up to a few gate/up items per workgroup, every gate/up item is
      // static: a claimed one could be queued behind the busy workgroup that
      // claimed it while an idle one takes a down item that waits for it
      // (1 row 36 -> 42 us, 64 Zipf rows 124 -> 134 us with the last
      // half-round claimed).  From 6 per workgroup on (384 rows: 8), the
      // last half-round of them is claimed, so the workgroups that finish
      // their static items first take it (384 rows 423.7 -> 405.7 us).
      // Every workgroup computes the same S: it depends on the routing only.
      i_dyn = i_rgu_end - p.i_pre_end >= 6 * G ? max(p.i_pre_end, min(i_rgu_end, i_total - G) - G / 2)
                                               : max(i_rgu_end, i_total - G);
      if (it >= i_dyn) {        // past the static part: claim (blocking, once)
        dyn = true;
        if (tid == 0) L.misc[2] = i_dyn + cgroup + kClaimGroups * atomic_add_agent(claim_ctr(), 1);
        __syncthreads();
        it = __builtin_amdgcn_readfirstlane(L.misc[2]);
        __syncthreads();
      }
    }
    const bool claim = routed && (dyn || it + G >= i_dyn);
    int claimed = 0;              // raw counter value; read only after the item
    if (tid == 0 && claim) claimed = atomic_add_agent(claim_ctr(), 1);
    t_got = t_ready = tl_clock(p);
    if (it < p.i_router_end) {
      kind = 0;
      if (NORM && !FULL && p.router_tiles) {
        // the router tile's rows of xn (small router items wait inside,
        // after requesting their first weights)
        const int n_et = (p.E + kRouterTile - 1) / kRouterTile;
        const int t0 = (it / p.router_ks / n_et) * kRouterTile;
        if (!rows_all && !wait_rows(p, L, t0, min(kRouterTile, p.T - t0))) break;
      }
      if (!FULL && p.router_tiles) {
        if constexpr (!FULL) router_tile_item(p, L, it);
      } else {
        // a small batch's router item reads all of x: it fills the LDS copy too
        const bool stage = !x_staged && p.T <= kRouterRows;
        t_ready = router_item<NORM>(p, L, it, stage);
        if (NORM && t_ready == LLONG_MIN) break;
        x_staged = x_staged || stage;
      }
    } else if (it >= p.i_topk_end && it < p.i_pre_end) {
      kind = 1;
      if (!ensure_x()) break;
      const int i = it - p.i_topk_end;
      const int mr = i / p.n_gu_mr, rb = i % p.n_gu_mr;
      const int r0 = mr * p.mrange;
      if constexpr (NORM && !XL)
        if (!rows_all && !wait_rows(p, L, r0, min(p.mrange, p.T - r0))) break;
      run_gu(p.E, p.T * p.K, r0, min(p.mrange, p.T - r0), rb, true);
    } else if (!FULL && it < p.i_topk_end) {
      kind = 2;
      if (!topk_item(p, L, it - p.i_router_end)) break;
      t_ready = *(SHARED long long*)(L.misc + 12);
      publish_done(L.ctr + kCtrTopkDone, p.n_topk, L.ctr + kCtrTopkGo);
    } else {
      kind = 6;
      if (!ensure_x()) break;
      if (!ensure_routing()) break;
      t_ready = tl_clock(p);
      if (it >= i_total) break;
      if (it < i_rgu_end) {
        kind = 4;
        if constexpr (NORM && !XL) {
          if (!rows_all) {
            if (!wait_rows(p, L, 0, p.T)) break;
            rows_all = true;
          }
        }
        const int i = it - p.i_pre_end;
        const int m = i / p.n_gu_mr, rb = i % p.n_gu_mr;
        const int e = L.mrlist[m];
        const int r0 = (m - L.nmrb[e]) * p.mrange;
        run_gu(e, L.base[e], r0, min(p.mrange, L.cnt[e] - r0), rb, false);
      } else if (it < i_rdn_end) {
        // down items.  Wide items go column group by column group (all
        // M-ranges of a 512-row group, shared first), so a group's combine
        // items find it complete while later groups still stream; otherwise
        // the shared M-ranges come first, then the routed ones, each
        // M-range's groups together.
        const int i = it - i_rgu_end;
        int mm, rg;
        if (p.wide) {
          const int nm = p.n_mr_sh + n_mr;
          rg = i / nm;
          mm = i - rg * nm;
        } else {
          const int j = i < p.n_sdn ? i : i - p.n_sdn;
          mm = j / p.n_dn_mr + (i < p.n_sdn ? 0 : p.n_mr_sh);
          rg = j % p.n_dn_mr;
        }
        int slot, sbase, r0, rows;
        if (mm < p.n_mr_sh) {
          kind = 3;
          slot = p.E;
          sbase = p.T * p.K;
          r0 = mm * p.mrange;
          rows = p.T;
        } else {
          kind = 5;
          const int m = mm - p.n_mr_sh;
          const int e = L.mrlist[m];
          slot = e;
          sbase = L.base[e];
          r0 = (m - L.nmrb[e]) * p.mrange;
          rows = L.cnt[e];
        }
        if (!run_down(slot, sbase, r0, min(p.mrange, rows - r0), rg, h_target(rows))) break;
        t_ready = *(SHARED long long*)(L.misc + 12);
      } else {
        kind = 7;
        flush_pending_now(L.ctr, pend_rg);
        // combine items: by column group for wide items (the order their
        // down items complete in), else by row group
        const int c = it - i_rdn_end;
        const int n_rc = (p.T + p.cmb_rows - 1) / p.cmb_rows;
        const int rc = p.wide ? c % n_rc : c / p.n_rg, rg = p.wide ? c / n_rc : c % p.n_rg;
        bool ok;
        if constexpr (WIDE) {
          ok = p.cmb_rows == 8 ? combine_item<4, 9, NORM>(p, L, rc, rg, n_mr)
                               : combine_item<2, kMaxTopK + 1, NORM>(p, L, rc, rg, n_mr);
        } else {
          ok = combine_item<2, kMaxTopK + 1, NORM>(p, L, rc, rg, n_mr);
        }
        if (!ok) break;
        t_ready = *(SHARED long long*)(L.misc + 12);
      }
    }
    record();
    if (kind == 2 && trace && tid == 0 && n_ev < p.trace_cap) {
      // a top-k item's gather: polling rounds, and when its first three ended
      long long* r = trace + (size_t)(1 + n_ev) * 4;
      st(r + 0, (long long)12 << 32 | (long long)min(L.misc[14], 0xffff));
      for (int i = 0; i < 3; ++i) st(r + 1 + i, i <= L.misc[14] ? ((SHARED long long*)(L.misc + 16))[i] : 0ll);
      ++n_ev;
    }
    if (claim) {
      // the claim's result is first read here, so the wait for its round
      // trip lands after the item (the empty asm keeps the compiler from
      // using it earlier); every item has a barrier after its last read of
      // misc[2]
      asm volatile("" : "+v"(claimed));
      if (tid == 0) L.misc[2] = i_dyn + cgroup + kClaimGroups * claimed;
      __syncthreads();
      it = __builtin_amdgcn_readfirstlane(L.misc[2]);
      dyn = true;
    } else {
      it += G;
    }
  }
  if (trace && tid == 0) {
    st(trace + 0, t_entry);
    st(trace + 1, (long long)wall_clock64());
    st(trace + 2, (long long)n_ev);
    st(trace + 3, (long long)G);
  }

  // a deferred column-group count still has to be given
  flush_pending_now(L.ctr, pend_rg);
}

// ----------------------------------------------------------------------------
// Weight re-layout (create time): standard row-major weights and group-32
// scales -> 16 x 64 tiles of the format (WFmt).  Source rows: FP8 and MXFP8 one
// byte per element, MXFP4 two elements per byte (element 2j in the low nibble
// of byte j); scales [rows][K/32] fp32 (FP8) or E8M0 bytes (MX).  For the
// gate/up matrix row block rb holds gate rows 8 rb .. 8 rb + 7 then up rows
// I + 8 rb .. I + 8 rb + 7.  An intermediate width I that is a multiple of 32
// but not of 64 is padded to the next multiple of 64 (I_p): the padding
// gate and up rows and the padding down-projection columns get zero weights
// and zero scales (E8M0 byte 0), so their g, u and h are exactly 0 and they
// add nothing to any sum ("Beyond Day-0: Optimizing DeepSeek-V4.1 Flash in
// SGLang", section 3.1: the per-GPU width 288 of TP8 is padded to 320 after
// sharding).
//   rows_p, K_p   : packed rows and K (multiples of 16 and 64)
//   rows_s, K_s   : the caller's rows and K (K_s a multiple of 32)
//   half_p, half_s: gate/up matrix: I_p and I (0 for the down projection)
// ----------------------------------------------------------------------------
template <int FMT>
__global__ void pack_kernel(const uint8_t* __restrict__ w, const void* __restrict__ s,
                            void* __restrict__ wp, void* __restrict__ sp, int slots, int rows_p,
                            int K_p, int rows_s, int K_s, int half_p, int half_s) {
  using Sc = typename WFmt<FMT>::Scale;
  const int nrb = rows_p / kTileRows, nq = K_p / kTileK, G_s = K_s / kGroup;
  const size_t row_bytes = FMT == kFmtMxfp4 ? (size_t)K_s / 2 : (size_t)K_s;
  const size_t total = (size_t)slots * nrb * nq * kWave;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(i % kWave);
    const size_t tile = i / kWave;
    const int q = (int)(tile % nq);
    const size_t blk = tile / nq;
    const int rb = (int)(blk % nrb);
    const int slot = (int)(blk / nrb);
    const int n = lane & 15, kq = lane >> 4;
    int row;
    bool rvalid = true;
    if (half_p > 0) {
      const int ii = 8 * rb + (n & 7);       // intermediate column of this gate or up row
      rvalid = ii < half_s;
      row = n < 8 ? ii : half_s + ii;
    } else {
      row = kTileRows * rb + n;
    }
    const size_t r_s = (size_t)slot * rows_s + (rvalid ? row : 0);
    const uint8_t* src = w + r_s * row_bytes;
    uint32_t o[4];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int k = kTileK * q + kGroup * g + 8 * kq;   // this lane's 8 elements of group g
      const bool v = rvalid && k < K_s;
      if constexpr (FMT == kFmtMxfp4) {
        o[g] = v ? *(const uint32_t*)(src + k / 2) : 0u;
      } else {
        const u32x2 x = v ? *(const u32x2*)(src + k) : (u32x2){0u, 0u};
        o[2 * g] = x.x;
        o[2 * g + 1] = x.y;
      }
    }
    if constexpr (FMT == kFmtMxfp4) ((u32x2*)wp)[i] = (u32x2){o[0], o[1]};
    else ((u32x4*)wp)[i] = (u32x4){o[0], o[1], o[2], o[3]};
    if (kq == 0) {
      const int g0 = kTileK * q / kGroup;
      Sc* d = (Sc*)sp + tile * kTileRows + n;
      if constexpr (FMT == kFmtFp8) {
        const float* ss = (const float*)s + r_s * G_s;
        *d = (f32x2){rvalid && g0 < G_s ? ss[g0] : 0.f, rvalid && g0 + 1 < G_s ? ss[g0 + 1] : 0.f};
      } else {
        const uint8_t* ss = (const uint8_t*)s + r_s * G_s;
        uint32_t v = 0;
#pragma unroll
        for (int g = 0; g < 2; ++g) v |= (uint32_t)(rvalid && g0 + g < G_s ? ss[g0 + g] : 0) << (8 * g);
        *d = (Sc)v;
      }
    }
  }
}

// Router rows -> tiled copy for the router tiles (create time); experts past
// E are zero.
__global__ void pack_router_kernel(const float* __restrict__ w, f32x4* __restrict__ wt, int E, int H) {
  const int n_et = (E + kRouterTile - 1) / kRouterTile, ns = H / 16;
  const size_t total = (size_t)n_et * ns * kWave;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(i % kWave);
    const size_t st = i / kWave;
    const int step = (int)(st % ns), et = (int)(st / ns);
    const int e = kRouterTile * et + (lane & 15), k = 16 * step + 4 * (lane >> 4);
    wt[i] = e < E ? *(const f32x4*)(w + (size_t)e * H + k) : (f32x4){0.f, 0.f, 0.f, 0.f};
  }
}

// ----------------------------------------------------------------------------
// Workspace of moe_decode_run_static: counter blocks, status and arrival
// counters, logits, top-k, h and expert-output scratch of one run, in one
// array of fixed size that the code object provides (no allocation).  Each
// GPU holds its own copy, zero at load (static storage), for the life of the
// process; host code reaches it only through the address hipGetSymbolAddress
// returns for the current device.
// ----------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// ----------------------------------------------------------------------------
// Host side
// ----------------------------------------------------------------------------
size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Counter words of a workspace: two counter blocks, the status line, the
// arrival counters.
constexpr size_t kCtrWords = 2 * (size_t)kCtrHead + kLine + (size_t)kArriveGroups * kLine;

// Byte offsets of a run's workspace in the static array (for T rows on a
// handle's shape): the same buffers create() allocates, sized for T.
struct StaticLayout {
  size_t ctr, lgt, topk_idx, topk_w, h_scr, o_scr, total;
};
StaticLayout static_layout(const moe_decode_config& c, int I_p, int T) {
  const size_t E = c.num_experts, H = c.hidden, K = c.top_k, S = c.num_shared;
  const size_t rows = (size_t)T * (K + S);
  StaticLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes, 256); return o; };
  L.ctr = take(kCtrWords * 4);
  L.lgt = take(std::max((size_t)T * E * kRouterKsMax, (size_t)kLgCopies * E * 16) * 8);
  L.topk_idx = take((size_t)T * K * 4);
  L.topk_w = take((size_t)T * K * 4);
  L.h_scr = take(rows * (I_p / 2) * 8);
  L.o_scr = take(rows * H * 8);
  L.total = off;
  return L;
}

// The static array's device address, per device, looked up once (with the
// device current).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
unsigned char* g_scratch_ptr[kMaxDevices] = {};
moe_status scratch_address(int device, unsigned char** out) {
  if (device < 0 || device >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_ERR_HIP;
    g_scratch_ptr[device] = (unsigned char*)ptr;
  }
  *out = g_scratch_ptr[device];
  return MOE_OK;
}

}  // namespace

struct moe_decode_handle {
  moe_decode_config cfg;
  int device;
  int n_cu;
  int coop;
  float* router_w = nullptr;
  f32x4* router_wt = nullptr;
  float* router_b = nullptr;
  int fmt = kFmtFp8;              // expert weight format (config flags)
  void* w13p = nullptr;
  void* s13p = nullptr;
  void* w2p = nullptr;
  void* s2p = nullptr;
  size_t w13_bytes = 0, s13_bytes = 0, w2_bytes = 0, s2_bytes = 0;
  uint64_t* lgt = nullptr;
  size_t lgt_bytes = 0;   // tile path: [ks][T][E]; small batches: [copy][E][8 or 16]
  int* topk_idx = nullptr;
  float* topk_w = nullptr;
  uint64_t* h_scr = nullptr;
  uint64_t* o_scr = nullptr;
  int* ctr = nullptr;
  // pre-norm block runs (moe_decode_set_input_norm)
  float* norm_w = nullptr;       // [H]
  uint16_t* xn = nullptr;        // [max_tokens][H] bf16
  int* norm_ready = nullptr;     // [max_tokens]
  float norm_eps = 0.f;
  float swiglu_limit = INFINITY; // moe_decode_set_swiglu_limit
  hipEvent_t ev_start = nullptr;  // moe_decode_set_launch_events
  hipEvent_t ev_stop = nullptr;
  hipStream_t last_stream = nullptr;
  int* last_status = nullptr;    // status word of the last run's workspace (handle's or static)
  std::mutex mu;
  // occupancy cache, by (kernel variant + 8 for paired gate/up items + 16 for
  // block runs, LDS bytes); occ_lds starts at -1 (set in create)
  int occ_lds[32];
  int occ_blocks[32] = {};
};

namespace {

// Expert weight format of a config (its flags' low two bits).
int weight_format(const moe_decode_config& c) { return (int)(c.flags & 3u); }

moe_status check_config(const moe_decode_config* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if ((c->flags & ~(3u | MOE_FLAG_COOPERATIVE)) != 0 || weight_format(*c) == 3 || c->deadline_us < 0)
    return MOE_ERR_INVALID_ARG;
  if (c->max_tokens < 1 || c->hidden < 1 || c->num_experts < 1 || c->top_k < 1 ||
      c->intermediate < 1 || c->num_shared < 0)
    return MOE_ERR_INVALID_ARG;
  if (c->max_tokens > kMaxTokens) return MOE_ERR_UNSUPPORTED;
  if (c->hidden % kTileK != 0 || c->hidden > 16384) return MOE_ERR_UNSUPPORTED;
  if (c->intermediate % kGroup != 0 || c->intermediate > 8192) return MOE_ERR_UNSUPPORTED;
  if (c->num_experts > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (c->top_k > kMaxTopK || c->top_k > c->num_experts) return MOE_ERR_UNSUPPORTED;
  if (c->num_shared > 1) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// The intermediate width the kernel runs: I rounded up to whole 64-K tiles
// (the padding is zero weights, see pack_kernel).
int padded_intermediate(const moe_decode_config& c) { return (c.intermediate + kTileK - 1) / kTileK * kTileK; }

Params make_params(const moe_decode_handle* h, int T) {
  const moe_decode_config& c = h->cfg;
  Params p;
  memset(&p, 0, sizeof(p));
  p.T = T;
  p.H = c.hidden;
  p.E = c.num_experts;
  p.K = c.top_k;
  p.S = c.num_shared;
  p.I = padded_intermediate(c);
  p.router_w = h->router_w;
  p.router_wt = h->router_wt;
  p.router_b = h->router_b ? h->router_b : h->router_w;
  p.has_bias = h->router_b != nullptr;
  p.w13p = h->w13p;
  p.s13p = h->s13p;
  p.w2p = h->w2p;
  p.s2p = h->s2p;
  p.w13_bytes = h->w13_bytes;
  p.s13_bytes = h->s13_bytes;
  p.w2_bytes = h->w2_bytes;
  p.s2_bytes = h->s2_bytes;
  p.lgt = h->lgt;
  p.lg_copies = kLgCopies;
  p.lg_tp_log2 = T <= 8 ? 3 : 4;
  p.fd_x8 = make_fdiv((uint32_t)(p.H / 8));
  p.fd_h2 = make_fdiv((uint32_t)(p.I / 2));
  p.fd_k = make_fdiv((uint32_t)p.K);
  p.topk_idx = h->topk_idx;
  p.topk_w = h->topk_w;
  p.h_scr = h->h_scr;
  p.o_scr = h->o_scr;
  p.ctr_base = h->ctr;
  p.status = h->ctr + 2 * (size_t)kCtrHead;
  p.arrive = (unsigned long long*)(h->ctr + 2 * (size_t)kCtrHead + kLine);
  const long long dl = c.deadline_us > 0 ? c.deadline_us : 1000000;
  p.deadline_ticks = dl * 100;   // wall clock runs at 100 MHz
  p.swiglu_limit = h->swiglu_limit;
  p.router_tiles = T > kMBlock ? 1 : 0;
  p.local_topk = p.router_tiles ? 0 : 1;
  p.n_rb13 = p.I / 8;
  p.n_q13 = p.H / kTileK;
  p.n_rb2 = p.H / kTileRows;
  p.n_q2 = p.I / kTileK;
  p.n_rg = (p.H + kDownRows - 1) / kDownRows;
  p.nch = (T + 63) / 64;
  p.wide = T > kMBlock && p.n_q13 == kWaves * kWideTiles &&
           p.n_q2 >= kWideQ2 && p.n_q2 <= kWideQ2 + 2;
  p.mrange = p.wide ? kWideRows : kMRange;
  // The full-tile variant: x and h in LDS (at most 16 rows), H = 64 kFullTiles,
  // I = 32 kFullTiles or 576, local routing.  With MXFP4 weights its gate/up
  // items cover two row blocks, so a wave has as many bytes in flight as with
  // FP8 tiles (the items are bound by latency, not by bytes), when that still
  // leaves at least two items per workgroup (the grid holds two per compute
  // unit) for as many experts as the call can touch: at 1 row the 288 paired
  // items would leave half the grid idle (measured slower, 34.4 -> 38.1 us).
  p.full = !p.wide && T <= kMBlock && (size_t)T * (p.H + 8) * 2 <= kXsMaxBytes && p.I <= kHsMaxI &&
           p.n_q13 == 4 * kFullTiles && (p.n_q2 == kFullTiles / 2 || p.n_q2 == kFullTiles / 2 + 1);
  const long long max_experts = std::min((long long)T * p.K, (long long)p.E) + p.S;
  p.gu_pair = p.full && h->fmt == kFmtMxfp4 && max_experts * (p.n_rb13 / 2) >= 2LL * 2 * h->n_cu;
  p.n_gu_mr = p.wide ? p.n_rb13 / kWideRb : p.gu_pair ? p.n_rb13 / 2 : p.n_rb13;
  p.n_dn_mr = p.wide ? p.H / (kWaves * kWideDnBlocks * kTileRows) : p.n_rg;
  p.h_rows_per_count = p.wide ? kWideRows : kMBlock;
  p.n_mr_sh = p.S ? (T + p.mrange - 1) / p.mrange : 0;
  {
    const int n_tiles = ((T + kRouterTile - 1) / kRouterTile) * ((p.E + kRouterTile - 1) / kRouterTile);
    // split H until the tiles make up to about two items per workgroup (the
    // top-k items then add ks partial logits); each wave's share of H must
    // stay a multiple of 16
    int ks = 1;
    while (2 * ks <= kRouterKsMax && n_tiles * 2 * ks <= 1024 && (p.H / kTileK) % (2 * ks) == 0) ks *= 2;
    p.router_ks = p.router_tiles ? ks : 1;
    p.n_router = p.router_tiles ? n_tiles * p.router_ks : p.E * ((T + kRouterRows - 1) / kRouterRows);
  }
  p.n_topk = p.local_topk ? 0 : (T + kWaves - 1) / kWaves;
  p.i_router_end = p.n_router;
  p.i_topk_end = p.i_router_end + p.n_topk;
  p.i_pre_end = p.i_topk_end + p.n_mr_sh * p.n_gu_mr;
  p.n_sdn = p.n_mr_sh * p.n_dn_mr;
  // larger combine items once the 4-row ones outnumber the workgroups about
  // twice (fewer latency-bound items in the tail); below that the items
  // would not fill the grid
  p.cmb_rows = p.wide && p.K <= 8 && T >= 128 ? 8 : kCombineRows;
  p.n_cmb = (T + p.cmb_rows - 1) / p.cmb_rows * p.n_rg;
  // LDS layout
  const int E = p.E, K = p.K;
  const int max_mr = E + (T * K + p.mrange - 1) / p.mrange;
  const int nmb = T > kMBlock ? 4 : p.gu_pair ? 2 : 1;   // MFMA blocks (or row blocks) of partial sums
  size_t off = 0;
  auto take = [&](size_t bytes) __attribute__((always_inline)) { size_t o = off; off = align_up(off + bytes, 16); return (int)o; };
  if (p.wide) {
    // one area used in turn by the placement bitmaps, the partial sums of
    // router tiles and gate/up items, the top-k items' logits and a down
    // item's h rows (each user is separated from the previous one by a
    // barrier); with it two workgroups fit on a compute unit
    p.hs_stride = p.I + 8;
    const size_t bm_bytes = align_up((size_t)E * p.nch * 8, 16);
    const size_t u = std::max({bm_bytes + (size_t)E * p.nch * 4,
                               (size_t)kWaves * kWideRb * 2 * kWave * 16,
                               (size_t)kWideRows * p.hs_stride * 2,
                               (size_t)kWaves * p.router_ks * E * 4,
                               (size_t)kWaves * kWave * 16});
    const int ua = take(u);
    p.lds_bm = ua;
    p.lds_cp = ua + (int)bm_bytes;
    p.lds_red = p.lds_hs = p.lds_lg = ua;
  } else {
    p.lds_bm = take((size_t)E * p.nch * 8);
    p.lds_cp = take((size_t)E * p.nch * 4);
  }
  p.lds_cnt = take((size_t)E * 4);
  p.lds_base = take((size_t)E * 4);
  p.lds_nmrb = take((size_t)(E + 1) * 4);
  p.lds_mrlist = take((size_t)max_mr * 4);
  p.lds_rows = take((size_t)T * K * 2);
  p.lds_tki = take((size_t)T * K * 2);
  p.lds_prow = take((size_t)T * K * 2);
  p.lds_tkw = take((size_t)T * K * 4);
  p.lds_misc = take(32 * 4);
  p.lds_tks = take((size_t)kWaves * kWave * 4);
  if (!p.wide) {
    // small batches (every expert then has at most 16 rows: one MFMA block) keep
    // x in LDS (rows padded by 16 bytes against bank conflicts) and stage each
    // down item's h rows there as well
    const size_t xs_stride = (size_t)p.H + 8;
    if (T <= kMBlock && (size_t)T * xs_stride * 2 <= kXsMaxBytes) {
      p.xs_stride = (int)xs_stride;
      p.lds_xs = take((size_t)T * xs_stride * 2);
      if (p.I <= kHsMaxI) p.hs_stride = p.I + 8;
    }
    // partial sums of the router and of gate/up items (two alternating halves)
    p.lds_red = take((size_t)2 * kWaves * nmb * kWave * 16);
    // one region used in turn by the routing logits and a down item's h rows
    const size_t hs_bytes = p.hs_stride ? (size_t)std::min(T, kMBlock) * p.hs_stride * 2 : 0;
    const size_t lg_bytes = (size_t)(p.local_topk ? T : kWaves * p.router_ks) * E * 4;
    p.lds_hs = p.lds_lg = take(std::max(hs_bytes, lg_bytes));
  }
  p.lds_bytes = (int)off;
  return p;
}

#define HIP_TRY(x)                         \
  do {                                     \
    if ((x) != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

}  // namespace

extern "C" {

int32_t moe_decode_abi_version(void) { return MOE_DECODE_ABI_VERSION; }

const char* moe_decode_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_OUT_OF_MEMORY: return "out of device memory";
    case MOE_ERR_TIMEOUT: return "in-kernel wait passed its deadline";
    default: return "unknown status";
  }
}

moe_status moe_decode_supported(const moe_decode_config* cfg, int32_t T) {
  const moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (T > cfg->max_tokens) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

void moe_decode_destroy(moe_decode_handle* h) {
  if (!h) return;
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(h->device);
  (void)hipDeviceSynchronize();
  void* ptrs[] = {h->router_w, h->router_wt, h->router_b, h->w13p, h->s13p, h->w2p, h->s2p, h->lgt,
                  h->topk_idx, h->topk_w, h->h_scr, h->o_scr, h->ctr, h->norm_w, h->xn, h->norm_ready};
  for (void* q : ptrs)
    if (q) (void)hipFree(q);
  (void)hipSetDevice(prev);
  delete h;
}

moe_status moe_decode_create(const moe_decode_config* cfg, const moe_decode_weights* w,
                             int32_t device, moe_decode_handle** out) {
  if (!out) return MOE_ERR_INVALID_ARG;
  *out = nullptr;
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (!w || !w->router_w || !w->w13 || !w->s13 || !w->w2 || !w->s2) return MOE_ERR_INVALID_ARG;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess) return MOE_ERR_HIP;
  if (device < 0 || device >= ndev) return MOE_ERR_INVALID_ARG;
  int prev = 0;
  HIP_TRY(hipGetDevice(&prev));
  HIP_TRY(hipSetDevice(device));

  moe_decode_handle* h = new (std::nothrow) moe_decode_handle();
  if (!h) return MOE_ERR_OUT_OF_MEMORY;
  h->cfg = *cfg;
  h->device = device;
  h->fmt = weight_format(*cfg);
  for (int& v : h->occ_lds) v = -1;
  moe_status rc = MOE_OK;
  do {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) { rc = MOE_ERR_HIP; break; }
    h->n_cu = prop.multiProcessorCount;
    h->coop = prop.cooperativeLaunch;
    if ((cfg->flags & MOE_FLAG_COOPERATIVE) && !h->coop) { rc = MOE_ERR_UNSUPPORTED; break; }
    // I: the packed (padded) width; I_s: the caller's
    const size_t E = cfg->num_experts, S = cfg->num_shared, H = cfg->hidden,
                 I = padded_intermediate(*cfg), I_s = cfg->intermediate, K = cfg->top_k, Tm = cfg->max_tokens;
    const size_t slots = E + S;
    const size_t scr_rows = Tm * K + Tm * S;
    // packed weights: FP8 and MXFP8 one byte per element, MXFP4 half a byte;
    // scales one fp32 (FP8) or one E8M0 byte (MX) per 32 elements
    const size_t w_num = h->fmt == kFmtMxfp4 ? 1 : 2, s_bytes = h->fmt == kFmtFp8 ? 4 : 1;
    h->w13_bytes = slots * 2 * I * H * w_num / 2;
    h->s13_bytes = slots * 2 * I * (H / 32) * s_bytes;
    h->w2_bytes = slots * H * I * w_num / 2;
    h->s2_bytes = slots * H * (I / 32) * s_bytes;
    // two counter blocks, the status line, the arrival counters
    const size_t ctr_words = kCtrWords;
    struct A { void** p; size_t bytes; } allocs[] = {
        {(void**)&h->router_w, E * H * 4},
        {(void**)&h->router_b, w->router_bias ? E * 4 : 0},
        {(void**)&h->w13p, h->w13_bytes},
        {(void**)&h->s13p, h->s13_bytes},
        {(void**)&h->w2p, h->w2_bytes},
        {(void**)&h->s2p, h->s2_bytes},
        {(void**)&h->lgt, h->lgt_bytes = std::max(Tm * E * kRouterKsMax, (size_t)kLgCopies * E * 16) * 8},
        {(void**)&h->topk_idx, Tm * K * 4},
        {(void**)&h->topk_w, Tm * K * 4},
        {(void**)&h->h_scr, scr_rows * (I / 2) * 8},
        {(void**)&h->o_scr, scr_rows * H * 8},
        {(void**)&h->ctr, ctr_words * 4},
        // tiled router rows, only for handles that can run router tiles
        {(void**)&h->router_wt, Tm > (size_t)kMBlock ? (E + kRouterTile - 1) / kRouterTile * kRouterTile * H * 4 : 0},
    };
    for (auto& a : allocs) {
      if (a.bytes == 0) continue;
      if (hipMalloc(a.p, a.bytes) != hipSuccess) { rc = MOE_ERR_OUT_OF_MEMORY; break; }
    }
    if (rc != MOE_OK) break;
    // counters and every tagged word start at zero (no run has epoch 0)
    if (hipMemset(h->ctr, 0, ctr_words * 4) != hipSuccess ||
        hipMemset(h->lgt, 0, h->lgt_bytes) != hipSuccess ||
        hipMemset(h->h_scr, 0, scr_rows * (I / 2) * 8) != hipSuccess ||
        hipMemset(h->o_scr, 0, scr_rows * H * 8) != hipSuccess) { rc = MOE_ERR_HIP; break; }
    if (hipMemcpy(h->router_w, w->router_w, E * H * 4, hipMemcpyDeviceToDevice) != hipSuccess) { rc = MOE_ERR_HIP; break; }
    if (w->router_bias &&
        hipMemcpy(h->router_b, w->router_bias, E * 4, hipMemcpyDeviceToDevice) != hipSuccess) { rc = MOE_ERR_HIP; break; }
    if (h->router_wt) {
      hipLaunchKernelGGL(pack_router_kernel, dim3(1024), dim3(256), 0, 0, h->router_w, h->router_wt, (int)E, (int)H);
      if (hipGetLastError() != hipSuccess) { rc = MOE_ERR_HIP; break; }
    }
    auto pack = h->fmt == kFmtMxfp4 ? pack_kernel<kFmtMxfp4> : h->fmt == kFmtMxfp8 ? pack_kernel<kFmtMxfp8>
                                                                                  : pack_kernel<kFmtFp8>;
    hipLaunchKernelGGL(pack, dim3(4096), dim3(256), 0, 0, w->w13, w->s13, h->w13p, h->s13p,
                       (int)slots, (int)(2 * I), (int)H, (int)(2 * I_s), (int)H, (int)I, (int)I_s);
    if (hipGetLastError() != hipSuccess) { rc = MOE_ERR_HIP; break; }
    hipLaunchKernelGGL(pack, dim3(4096), dim3(256), 0, 0, w->w2, w->s2, h->w2p, h->s2p,
                       (int)slots, (int)H, (int)I, (int)H, (int)I_s, 0, 0);
    if (hipGetLastError() != hipSuccess) { rc = MOE_ERR_HIP; break; }
    if (hipDeviceSynchronize() != hipSuccess) { rc = MOE_ERR_HIP; break; }
  } while (0);
  (void)hipSetDevice(prev);
  if (rc != MOE_OK) {
    moe_decode_destroy(h);
    return rc;
  }
  *out = h;
  return MOE_OK;
}

}  // extern "C"

namespace {

// The kernel of a variant (see run_impl) for weight format FMT.  pair: the
// full-tile MXFP4 kernel with paired gate/up items (variants 3 and 5 only).
template <int FMT>
const void* kernel_for(int variant, bool norm, bool pair = false) {
  constexpr int q = kFullTiles / 2;   // down tiles per row block at I = 32 kFullTiles
  if constexpr (FMT == kFmtMxfp4) {
    if (pair && (variant == 3 || variant == 5)) {
      if (variant == 3)
        return norm ? (const void*)moe_decode_kernel<1, true, true, false, q, true, FMT, true>
                    : (const void*)moe_decode_kernel<1, true, true, false, q, false, FMT, true>;
      return norm ? (const void*)moe_decode_kernel<1, true, true, false, q + 1, true, FMT, true>
                  : (const void*)moe_decode_kernel<1, true, true, false, q + 1, false, FMT, true>;
    }
  }
  if (pair) return nullptr;
  if (variant == 4 || variant == 6 || variant == 7) {
    if (variant == 6)
      return norm ? (const void*)moe_decode_kernel<2, false, false, true, kWideQ2 + 1, true, FMT>
                  : (const void*)moe_decode_kernel<2, false, false, true, kWideQ2 + 1, false, FMT>;
    else if (variant == 7)
      return norm ? (const void*)moe_decode_kernel<2, false, false, true, kWideQ2 + 2, true, FMT>
                  : (const void*)moe_decode_kernel<2, false, false, true, kWideQ2 + 2, false, FMT>;
    else return norm ? (const void*)moe_decode_kernel<2, false, false, true, kWideQ2, true, FMT>
                     : (const void*)moe_decode_kernel<2, false, false, true, kWideQ2, false, FMT>;
  }
  if (norm) {
    switch (variant) {
      case 3: return (const void*)moe_decode_kernel<1, true, true, false, q, true, FMT>;
      case 5: return (const void*)moe_decode_kernel<1, true, true, false, q + 1, true, FMT>;
      case 0: return (const void*)moe_decode_kernel<1, true, false, false, q, true, FMT>;
      case 1: return (const void*)moe_decode_kernel<1, false, false, false, q, true, FMT>;
      default: return (const void*)moe_decode_kernel<4, false, false, false, q, true, FMT>;
    }
  }
  switch (variant) {
    case 3: return (const void*)moe_decode_kernel<1, true, true, false, q, false, FMT>;
    case 5: return (const void*)moe_decode_kernel<1, true, true, false, q + 1, false, FMT>;
    case 0: return (const void*)moe_decode_kernel<1, true, false, false, q, false, FMT>;
    case 1: return (const void*)moe_decode_kernel<1, false, false, false, q, false, FMT>;
    default: return (const void*)moe_decode_kernel<4, false, false, false, q, false, FMT>;
  }
}

// One layer call (norm = false) or pre-norm block call (norm = true).
moe_status run_impl(moe_decode_handle* h, const void* x, int32_t T, void* y,
                    const moe_decode_debug* dbg, void* hip_stream, bool norm, bool in_static = false) {
  if (!h) return MOE_ERR_INVALID_ARG;
  if (norm && !h->xn) return MOE_ERR_INVALID_ARG;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (T > h->cfg.max_tokens) return MOE_ERR_UNSUPPORTED;   // as the Guard answers for it
  if (T == 0) return MOE_OK;
  if (!x || !y) return MOE_ERR_INVALID_ARG;
  if (((uintptr_t)x | (uintptr_t)y) & 15u) return MOE_ERR_INVALID_ARG;
  const size_t bytes = (size_t)T * h->cfg.hidden * 2;
  const uintptr_t xa = (uintptr_t)x, ya = (uintptr_t)y;
  if (xa < ya + bytes && ya < xa + bytes) return MOE_ERR_INVALID_ARG;

  Params p = make_params(h, T);
  p.x = (const uint16_t*)x;
  p.y = (uint16_t*)y;
  if (norm) {
    p.x_in = (const uint16_t*)x;
    p.x = h->xn;
    p.xn = h->xn;
    p.norm_w = h->norm_w;
    p.norm_ready = h->norm_ready;
    p.norm_eps = h->norm_eps;
    if (dbg) p.dbg_norm = (uint16_t*)dbg->norm_x;
  }
  if (dbg) {
    p.dbg_idx = dbg->topk_idx;
    p.dbg_w = dbg->topk_w;
    p.dbg_rank = dbg->pair_rank;
    p.dbg_count = dbg->expert_count;
    p.dbg_logits = dbg->logits;
    p.expire_waits = dbg->expire_waits != 0;
    if (dbg->trace && dbg->trace_blocks > 0 && dbg->trace_cap > 0) {
      p.trace = (long long*)dbg->trace;
      p.trace_blocks = dbg->trace_blocks;
      p.trace_cap = dbg->trace_cap;
    }
  }
  hipStream_t stream = (hipStream_t)hip_stream;
  std::lock_guard<std::mutex> lock(h->mu);
  int prev = 0;
  HIP_TRY(hipGetDevice(&prev));
  if (prev != h->device) HIP_TRY(hipSetDevice(h->device));
  if (in_static) {
    // the whole workspace in the static array of this device
    const StaticLayout sl = static_layout(h->cfg, p.I, T);
    unsigned char* base = nullptr;
    moe_status st = sl.total > kScratchBytes ? MOE_ERR_UNSUPPORTED : scratch_address(h->device, &base);
    if (st != MOE_OK) {
      if (prev != h->device) (void)hipSetDevice(prev);
      return st;
    }
    int* ctr = (int*)(base + sl.ctr);
    p.ctr_base = ctr;
    p.status = ctr + 2 * (size_t)kCtrHead;
    p.arrive = (unsigned long long*)(ctr + 2 * (size_t)kCtrHead + kLine);
    p.lgt = (uint64_t*)(base + sl.lgt);
    p.topk_idx = (int*)(base + sl.topk_idx);
    p.topk_w = (float*)(base + sl.topk_w);
    p.h_scr = (uint64_t*)(base + sl.h_scr);
    p.o_scr = (uint64_t*)(base + sl.o_scr);
  }
  // variants: 0 = x in LDS, 1 = up to 16 rows, 2 = more rows (4 MFMA blocks
  // per item), 3 = x in LDS with full-tile items (H = 64 kFullTiles,
  // I = 32 kFullTiles, h staged in LDS, local routing), 5 = the same with one
  // more down tile per row block (I = 576 at 64-K tiles: the pages' per-GPU
  // width without padding), 4 = more than 16 rows with wide items
  // (H = 64 kWideTiles, I = 64 kWideQ2), 6 and 7 = the same at I = 576 and 640
  // (one and two more down K tiles per row block)
  const bool full = p.full != 0;
  // paired gate/up items exist only in the full-tile MXFP4 kernel, whose
  // list then holds n_rb13 / 2 of them per M-range and twice the partial-sum
  // area: refuse anything else before launching
  if ((p.gu_pair && (!full || h->fmt != kFmtMxfp4 || 2 * p.n_gu_mr != p.n_rb13)) ||
      (full && (p.xs_stride <= 0 || p.hs_stride <= 0))) {
    if (prev != h->device) (void)hipSetDevice(prev);
    return MOE_ERR_HIP;
  }
  const int variant = p.wide ? (p.n_q2 == kWideQ2 ? 4 : p.n_q2 == kWideQ2 + 1 ? 6 : 7)
                      : full ? (p.n_q2 == kFullTiles / 2 ? 3 : 5) : p.xs_stride > 0 ? 0 : (T > kMBlock ? 2 : 1);
  const void* fn = h->fmt == kFmtMxfp4   ? kernel_for<kFmtMxfp4>(variant, norm, p.gu_pair != 0)
                   : h->fmt == kFmtMxfp8 ? kernel_for<kFmtMxfp8>(variant, norm)
                                         : kernel_for<kFmtFp8>(variant, norm);
  if (!fn) {
    if (prev != h->device) (void)hipSetDevice(prev);
    return MOE_ERR_UNSUPPORTED;
  }
  const int slot = variant + (p.gu_pair ? 8 : 0) + (norm ? 16 : 0);
  if (h->occ_lds[slot] != p.lds_bytes) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, kThreads, p.lds_bytes) != hipSuccess ||
        nb < 1) {
      if (prev != h->device) (void)hipSetDevice(prev);
      return MOE_ERR_HIP;
    }
    h->occ_lds[slot] = p.lds_bytes;
    h->occ_blocks[slot] = nb;
  }
  const int grid = h->n_cu * h->occ_blocks[slot];
  if (grid < kArriveGroups || grid > (int)kRunUnits) {   // every arrival counter needs a workgroup each run
    if (prev != h->device) (void)hipSetDevice(prev);
    return MOE_ERR_UNSUPPORTED;
  }
  // The grid is sized to what the device holds at once, so all workgroups
  // are resident together on an otherwise idle device; every wait has a
  // deadline for the case where they are not, and MOE_FLAG_COOPERATIVE makes
  // the runtime guarantee it (or refuse the launch).
  void* args[] = {&p};
  const bool coop = (h->cfg.flags & MOE_FLAG_COOPERATIVE) != 0;
  if (coop && h->ev_start) {                  // a cooperative launch takes no events
    if (prev != h->device) (void)hipSetDevice(prev);
    return MOE_ERR_UNSUPPORTED;
  }
  if (h->ev_start) {                          // launch events time eager runs only
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    const hipError_t qe = hipStreamIsCapturing(stream, &cs);
    if (qe != hipSuccess || cs != hipStreamCaptureStatusNone) {
      if (prev != h->device) (void)hipSetDevice(prev);
      return qe != hipSuccess ? MOE_ERR_HIP : MOE_ERR_UNSUPPORTED;
    }
  }
  const hipError_t err =
      coop ? hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kThreads), args, p.lds_bytes, stream)
      : h->ev_start
          ? hipExtLaunchKernel(fn, dim3(grid), dim3(kThreads), args, p.lds_bytes, stream, h->ev_start, h->ev_stop, 0)
          : hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, p.lds_bytes, stream);
  h->last_stream = stream;
  h->last_status = p.status;
  if (prev != h->device) (void)hipSetDevice(prev);
  return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace

extern "C" {

moe_status moe_decode_run(moe_decode_handle* h, const void* x, int32_t T, void* y,
                          const moe_decode_debug* dbg, void* hip_stream) {
  return run_impl(h, x, T, y, dbg, hip_stream, false);
}

moe_status moe_decode_run_static(moe_decode_handle* h, const void* x, int32_t T, void* y,
                                 const moe_decode_debug* dbg, void* hip_stream) {
  return run_impl(h, x, T, y, dbg, hip_stream, false, true);
}

moe_status moe_decode_set_input_norm(moe_decode_handle* h, const float* norm_w, float eps) {
  if (!h || !norm_w || !(eps > 0.f && eps < 1e30f)) return MOE_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(h->mu);
  int prev = 0;
  HIP_TRY(hipGetDevice(&prev));
  if (prev != h->device) HIP_TRY(hipSetDevice(h->device));
  moe_status rc = MOE_OK;
  const size_t H = h->cfg.hidden, Tm = h->cfg.max_tokens;
  do {
    // earlier runs may still read the weight being replaced
    if (h->last_stream != nullptr && hipStreamSynchronize(h->last_stream) != hipSuccess) { rc = MOE_ERR_HIP; break; }
    if (!h->xn) {
      if (hipMalloc((void**)&h->norm_w, H * 4) != hipSuccess ||
          hipMalloc((void**)&h->xn, Tm * H * 2) != hipSuccess ||
          hipMalloc((void**)&h->norm_ready, Tm * 4) != hipSuccess) {
        rc = MOE_ERR_OUT_OF_MEMORY;
      } else if (hipMemset(h->norm_ready, 0, Tm * 4) != hipSuccess) {
        rc = MOE_ERR_HIP;
      }
      if (rc != MOE_OK) {
        for (void* q : {(void*)h->norm_w, (void*)h->xn, (void*)h->norm_ready})
          if (q) (void)hipFree(q);
        h->norm_w = nullptr;
        h->xn = nullptr;
        h->norm_ready = nullptr;
        break;
      }
    }
    if (hipMemcpy(h->norm_w, norm_w, H * 4, hipMemcpyDeviceToDevice) != hipSuccess) { rc = MOE_ERR_HIP; break; }
    h->norm_eps = eps;
  } while (0);
  if (prev != h->device) (void)hipSetDevice(prev);
  return rc;
}

moe_status moe_decode_run_block(moe_decode_handle* h, const void* x, int32_t T, void* y,
                                const moe_decode_debug* dbg, void* hip_stream) {
  return run_impl(h, x, T, y, dbg, hip_stream, true);
}

moe_status moe_decode_set_swiglu_limit(moe_decode_handle* h, float limit) {
  if (!h || !(limit > 0.f)) return MOE_ERR_INVALID_ARG;   // NaN fails the test too
  std::lock_guard<std::mutex> lock(h->mu);
  h->swiglu_limit = limit;
  return MOE_OK;
}

moe_status moe_decode_set_launch_events(moe_decode_handle* h, void* start_event, void* stop_event) {
  if (!h || (start_event == nullptr) != (stop_event == nullptr)) return MOE_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(h->mu);
  h->ev_start = (hipEvent_t)start_event;
  h->ev_stop = (hipEvent_t)stop_event;
  return MOE_OK;
}

moe_status moe_decode_check(moe_decode_handle* h) {
  if (!h) return MOE_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(h->mu);
  int prev = 0;
  HIP_TRY(hipGetDevice(&prev));
  if (prev != h->device) HIP_TRY(hipSetDevice(h->device));
  moe_status rc = MOE_OK;
  int status = 0;
  int* const sw = h->last_status ? h->last_status : h->ctr + 2 * (size_t)kCtrHead;
  if (hipStreamSynchronize(h->last_stream) != hipSuccess ||
      hipMemcpy(&status, sw, 4, hipMemcpyDeviceToHost) != hipSuccess) {
    rc = MOE_ERR_HIP;
  } else if (status != 0) {
    rc = MOE_ERR_TIMEOUT;
    const int zero = 0;
    if (hipMemcpy(sw, &zero, 4, hipMemcpyHostToDevice) != hipSuccess) rc = MOE_ERR_HIP;
  }
  if (prev != h->device) (void)hipSetDevice(prev);
  return rc;
}

}  // extern "C"
