// Persistent MoE decode layer for MI355X (gfx950, CDNA4) behind the C ABI of
// include/moe_decode.h.
//
// One launch runs the whole layer.  Workgroups stay resident and pull work
// items from one ticket counter (an in-kernel queue); an item that needs the
// result of earlier items waits on a counter those items bump when done.  The
// idea of blocks that stay resident, hand ready results on through tagged
// buffers and keep at it across stages is the one described in "FlyDSL Mono
// Kernels for High-Interactivity LLM Serving in ATOM" (sections "What FlyDSL
// Provides" and "MiniMax-M3: Connecting Attention and Experts"); the deadline
// on every wait follows "SGLang's Low-Latency Mode Boosts DeepSeek-V4.1-Flash
// Speed by 1.56x on AMD" (section "AMD keeps the layer resident").
//
// Tickets, in this order (an item only ever waits on items with smaller
// tickets, which were taken by workgroups already running, so the queue makes
// progress whether or not every workgroup is resident):
//   router   : logits for 4 experts x 8 rows
//   shared gate/up (no routing needed), 16 weight rows (8 gate + 8 up)
//   top-k    : 4 rows, one per wave           -- waits: all router items
//   shared down, 128 output rows              -- waits: shared gate/up
//   routed gate/up, 16 weight rows per item   -- waits: all top-k items
//   routed down, 128 output rows per item     -- waits: that expert's gate/up
// The weighted combine runs in whichever down item arrives last for a
// (row, 128-column chunk).
//
// Expert weights are re-laid out once, at create time, into 1 KiB tiles of
// 16 weight rows x 64 K: lane l of a wave reads bytes [16 l, 16 l + 16) of a
// tile, i.e. every wave-wide load is one contiguous KiB.  Lane l = (n, kq),
// n = l % 16, kq = l / 16, holds row n's K elements [8 kq, 8 kq + 8) of the
// tile's first 32-element group and the same of its second group, which is
// exactly the B-operand layout of v_mfma_f32_16x16x32_bf16 for one group per
// instruction.  So one MFMA covers exactly one scale group: its fp32 result is
// multiplied by that group's scale and accumulated.  FP8 e4m3fn -> bf16 is
// exact (v_cvt_scalef32_pk_bf16_fp8 with scale 1), bf16 x bf16 products are
// exact in fp32, so the only rounding is fp32 accumulation.  The activation
// tile (up to 16 rows) is the A operand; rows beyond the expert's row count
// are zero.
#include <hip/hip_runtime.h>

#include <limits.h>
#include <stdint.h>
#include <string.h>

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
constexpr int kRouterRows = 8;              // rows per router item
constexpr int kDownRows = 128;              // output rows per down item (8 row blocks)
constexpr int kTileRows = 16;               // weight rows per tile
constexpr int kTileK = 64;                  // K elements per tile (two scale groups)
constexpr int kGroup = 32;
constexpr int kMaxTokens = 512;
constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 16;

// counter block
constexpr int kCtrTicket = 0;
constexpr int kCtrRouterDone = 1;
constexpr int kCtrTopkDone = 2;
constexpr int kCtrExit = 3;
constexpr int kCtrStatus = 4;
constexpr int kCtrHReady = 8;               // [E+S]

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct Params {
  int T, H, E, K, S, I;
  // inputs / outputs
  const uint16_t* x;
  uint16_t* y;
  const float* router_w;
  const float* router_b;
  const u32x4* w13p;   // [E+S][2I/16][H/64][64] tiles
  const float* s13p;   // [E+S][2I/16][H/64][16][2]
  const u32x4* w2p;    // [E+S][H/16][I/64][64]
  const float* s2p;    // [E+S][H/16][I/64][16][2]
  // workspace
  float* logits;       // [T][E]
  int* topk_idx;       // [T][K]
  float* topk_w;       // [T][K]
  uint16_t* h_scr;     // [T*K + T*S][I] bf16, rows grouped by expert
  float* o_scr;        // [T*K + T*S][H]
  int* ctr;            // counters
  int* pair_done;      // [T][n_rg]
  // debug copies (nullable)
  int* dbg_idx;
  float* dbg_w;
  int* dbg_rank;
  int* dbg_count;
  float* dbg_logits;
  // derived
  long long deadline_ticks;  // wall-clock ticks (100 MHz)
  int n_eb;            // router expert blocks: ceil(E/4)
  int n_rb13;          // gate/up row blocks per expert: I/8
  int n_q13;           // tiles along H: H/64
  int n_rb2;           // down row blocks: H/16
  int n_q2;            // tiles along I: I/64
  int n_rg;            // down row groups: ceil(H/128)
  int n_mr_sh;         // shared M-ranges: ceil(T/64) (0 without a shared expert)
  int nch;             // 64-row chunks: ceil(T/64)
  // ticket ranges [start, end)
  int t_router_end, t_sgu_end, t_topk_end, t_sdn_end;
  int n_router, n_topk;
  // LDS offsets (bytes)
  int lds_bm, lds_cp, lds_cnt, lds_base, lds_nmrb, lds_mrlist, lds_rows, lds_red, lds_comb, lds_misc;
  int lds_bytes;
};

// ----------------------------------------------------------------------------
// Small device helpers
// ----------------------------------------------------------------------------
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16, round to nearest even (overflow to inf, NaN kept NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

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

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, zero, 0, 0, 0);
}

__device__ __forceinline__ u32x4 load_nt(const u32x4* p) { return __builtin_nontemporal_load(p); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int atomic_add_agent(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int load_agent(int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fence_release_agent() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void fence_acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

// Thread 0 of the workgroup publishes "one more item done" on *ctr after
// every thread's stores of the item (barrier first, then an agent-scope
// release, then the increment).
__device__ void publish_done(int* ctr) {
  __syncthreads();
  if (threadIdx.x == 0) {
    fence_release_agent();
    atomic_add_agent(ctr, 1);
  }
}

// Workgroup-wide wait until *ctr >= target.  Thread 0 spins with a deadline;
// the result is broadcast through LDS.  false: deadline passed or another
// workgroup already reported an error -- the caller stops taking work.
__device__ bool wait_geq(const Params& p, int* ctr, int target, int* lds_flag) {
  if (threadIdx.x == 0) {
    int ok = 1;
    if (load_agent(ctr) < target) {
      const long long t_end = (long long)wall_clock64() + p.deadline_ticks;
      while (true) {
        if (load_agent(ctr) >= target) break;
        if (load_agent(p.ctr + kCtrStatus) != 0) { ok = 0; break; }
        if ((long long)wall_clock64() > t_end) {
          int expected = 0;
          __hip_atomic_compare_exchange_strong(p.ctr + kCtrStatus, &expected, MOE_ERR_TIMEOUT,
                                               __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    if (ok) fence_acquire_agent();
    *lds_flag = ok;
  }
  __syncthreads();
  int ok = *lds_flag;
  __syncthreads();
  return ok != 0;
}

// Block-wide exclusive prefix sum of one int per thread (kThreads values).
__device__ int block_exclusive_scan(int v, int* lds4, int* total) {
  const int lane = lane_id(), w = wave_id();
  int incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int n = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += n;
  }
  if (lane == kWave - 1) lds4[w] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    int s = lds4[i];
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
  unsigned long long* bm;  // [E][nch] row bitmap of each expert
  int* cp;                 // [E][nch] rows of the expert in earlier chunks
  int* cnt;                // [E] rows per expert
  int* base;               // [E] first scratch row of the expert
  int* nmrb;               // [E+1] prefix of M-ranges per expert
  int* mrlist;             // [n_mr] expert of each routed M-range
  int16_t* rows;           // [T*K] row -> token, grouped by expert
  float* red;              // [kWaves][4][64][4] partial sums
  int* comb;               // combine staging
  int* misc;               // [0] ticket, [1] flag, [2] n_mr, [3..7) scan scratch, [8] n_comb
};

__device__ Lds lds_view(const Params& p, char* smem) {
  Lds L;
  L.bm = (unsigned long long*)(smem + p.lds_bm);
  L.cp = (int*)(smem + p.lds_cp);
  L.cnt = (int*)(smem + p.lds_cnt);
  L.base = (int*)(smem + p.lds_base);
  L.nmrb = (int*)(smem + p.lds_nmrb);
  L.mrlist = (int*)(smem + p.lds_mrlist);
  L.rows = (int16_t*)(smem + p.lds_rows);
  L.red = (float*)(smem + p.lds_red);
  L.comb = (int*)(smem + p.lds_comb);
  L.misc = (int*)(smem + p.lds_misc);
  return L;
}

// Sort-free placement ("routing without sorting": each expert's rows go to
// 8-row tiles in row order, positions from a bitmap and population counts).
// Every pair (t, k) sets bit t of expert idx[t][k]'s bitmap; an expert's
// count is the popcount of its bitmap; a pair's rank is the popcount of the
// expert's bits below t.  Row r of expert e lives at scratch row base[e] + r.
__device__ void build_placement(const Params& p, const Lds& L) {
  const int tid = threadIdx.x;
  const int E = p.E, K = p.K, T = p.T, nch = p.nch;
  for (int i = tid; i < E * nch; i += kThreads) L.bm[i] = 0ull;
  __syncthreads();
  for (int i = tid; i < T * K; i += kThreads) {
    const int t = i / K;
    const int e = p.topk_idx[i];
    atomicOr(&L.bm[e * nch + (t >> 6)], 1ull << (t & 63));
  }
  __syncthreads();
  // counts, chunk prefixes, expert bases and M-range prefixes (E <= kThreads)
  int c = 0, nmr = 0;
  if (tid < E) {
    for (int ch = 0; ch < nch; ++ch) {
      L.cp[tid * nch + ch] = c;
      c += __popcll(L.bm[tid * nch + ch]);
    }
    L.cnt[tid] = c;
    nmr = (c + kMRange - 1) / kMRange;
  }
  int tot_rows, tot_mr;
  const int base = block_exclusive_scan(c, L.misc + 3, &tot_rows);
  const int mrb = block_exclusive_scan(nmr, L.misc + 3, &tot_mr);
  if (tid < E) {
    L.base[tid] = base;
    L.nmrb[tid] = mrb;
    for (int j = 0; j < nmr; ++j) L.mrlist[mrb + j] = tid;
  }
  if (tid == 0) {
    L.nmrb[E] = tot_mr;
    L.misc[2] = tot_mr;
  }
  __syncthreads();
  for (int i = tid; i < T * K; i += kThreads) {
    const int t = i / K;
    const int e = p.topk_idx[i];
    const unsigned long long below = L.bm[e * nch + (t >> 6)] & ((1ull << (t & 63)) - 1ull);
    const int rank = L.cp[e * nch + (t >> 6)] + __popcll(below);
    L.rows[L.base[e] + rank] = (int16_t)t;
  }
  __syncthreads();
}

// Rank of row t among expert e's rows -- valid after build_placement.
__device__ __forceinline__ int pair_rank(const Params& p, const Lds& L, int t, int e) {
  const unsigned long long below = L.bm[e * p.nch + (t >> 6)] & ((1ull << (t & 63)) - 1ull);
  return L.cp[e * p.nch + (t >> 6)] + __popcll(below);
}
__device__ __forceinline__ int pair_row(const Params& p, const Lds& L, int t, int e) {
  return L.base[e] + pair_rank(p, L, t, e);
}

// Optional debug copies of the placement (written by one workgroup).
__device__ void write_placement_debug(const Params& p, const Lds& L) {
  if (p.dbg_count)
    for (int e = threadIdx.x; e < p.E; e += kThreads) p.dbg_count[e] = L.cnt[e];
  if (p.dbg_rank)
    for (int i = threadIdx.x; i < p.T * p.K; i += kThreads)
      p.dbg_rank[i] = pair_rank(p, L, i / p.K, p.topk_idx[i]);
}

// ----------------------------------------------------------------------------
// Router: logits for 4 experts (one per wave) x up to 8 rows.
// ----------------------------------------------------------------------------
__device__ void router_item(const Params& p, int item) {
  const int w = wave_id(), lane = lane_id();
  const int e = (item % p.n_eb) * kWaves + w;
  const int t0 = (item / p.n_eb) * kRouterRows;
  const int nt = min(kRouterRows, p.T - t0);
  if (e < p.E) {
    float acc[kRouterRows];
#pragma unroll
    for (int j = 0; j < kRouterRows; ++j) acc[j] = 0.f;
    const float4* wr = (const float4*)(p.router_w + (size_t)e * p.H);
    const int n4 = p.H / 4;
    for (int c = lane; c < n4; c += kWave) {
      const float4 wv = wr[c];
#pragma unroll
      for (int j = 0; j < kRouterRows; ++j) {
        if (j < nt) {
          const u32x2 xv = *(const u32x2*)(p.x + (size_t)(t0 + j) * p.H + 4 * c);
          acc[j] += wv.x * bf16_to_f32(xv.x & 0xffffu) + wv.y * bf16_to_f32(xv.x >> 16) +
                    wv.z * bf16_to_f32(xv.y & 0xffffu) + wv.w * bf16_to_f32(xv.y >> 16);
        }
      }
    }
    const float b = p.router_b ? p.router_b[e] : 0.f;
#pragma unroll
    for (int j = 0; j < kRouterRows; ++j) {
      if (j < nt) {
        const float s = wave_sum(acc[j]) + b;
        if (lane == 0) {
          p.logits[(size_t)(t0 + j) * p.E + e] = s;
          if (p.dbg_logits) p.dbg_logits[(size_t)(t0 + j) * p.E + e] = s;
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Top-k: one row per wave.  Lane l holds experts l, l+64, l+128, l+192.
// Ranking by logit equals ranking by sigmoid score (monotone); ties go to the
// lower expert id.  Weights: sigmoid of the selected logits over their sum.
// ----------------------------------------------------------------------------
__device__ __forceinline__ int order_key(float v) {
  // order-preserving map of a float to an int; NaN sorts just above the
  // "unavailable" key so it can never displace a real score
  const int b = __float_as_int(v);
  if (v != v) return INT_MIN + 1;
  return b >= 0 ? b : (b ^ 0x7fffffff);
}

__device__ void topk_item(const Params& p, int item) {
  const int w = wave_id(), lane = lane_id();
  const int t = item * kWaves + w;
  if (t >= p.T) return;
  float v[4];
  int key[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + kWave * j;
    v[j] = e < p.E ? p.logits[(size_t)t * p.E + e] : 0.f;
    key[j] = e < p.E ? order_key(v[j]) : INT_MIN;   // INT_MIN: not selectable
  }
  int my_idx = 0;
  float my_logit = 0.f;
  for (int k = 0; k < p.K; ++k) {
    int bk = key[0], be = lane;
    float bv = v[0];
#pragma unroll
    for (int j = 1; j < 4; ++j) {
      if (key[j] > bk) { bk = key[j]; be = lane + kWave * j; bv = v[j]; }   // strict: lower id on ties
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const int ok = __shfl_xor(bk, o, kWave);
      const int oe = __shfl_xor(be, o, kWave);
      const float ov = __shfl_xor(bv, o, kWave);
      if (ok > bk || (ok == bk && oe < be)) { bk = ok; be = oe; bv = ov; }
    }
    if (lane == k) { my_idx = be; my_logit = bv; }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (be == lane + kWave * j) key[j] = INT_MIN;
  }
  const float s = lane < p.K ? 1.0f / (1.0f + __expf(-my_logit)) : 0.f;
  const float sum = wave_sum(s);
  if (lane < p.K) {
    const float wk = s / sum;
    p.topk_idx[t * p.K + lane] = my_idx;
    p.topk_w[t * p.K + lane] = wk;
    if (p.dbg_idx) p.dbg_idx[t * p.K + lane] = my_idx;
    if (p.dbg_w) p.dbg_w[t * p.K + lane] = wk;
  }
}

// ----------------------------------------------------------------------------
// Expert gate/up: one 16-row block (8 gate rows + 8 up rows) of one expert for
// up to 64 of its rows; the 4 waves split the H/64 tiles (wave w takes tiles
// q = w, w+4, ...); partial sums meet in LDS; then h = bf16(silu(g) * u).
// ----------------------------------------------------------------------------
template <int NMB>
__device__ void gu_item(const Params& p, const Lds& L, int slot, int sbase, int r0, int nrows,
                        int rb, bool shared) {
  const int w = wave_id(), lane = lane_id();
  const int n = lane & 15, kq = lane >> 4;
  const int nq = p.n_q13;
  const size_t blk = (size_t)slot * p.n_rb13 + rb;
  const u32x4* wt = p.w13p + blk * nq * kWave + lane;
  const float2* sc = (const float2*)p.s13p + blk * nq * kTileRows + n;

  // A operand rows: token of expert row r0 + mb*16 + n (zero when past nrows)
  const uint16_t* arow[NMB];
  bool aval[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    const int r = mb * kMBlock + n;
    aval[mb] = r < nrows;
    int tok = 0;
    if (aval[mb]) tok = shared ? (r0 + r) : (int)L.rows[sbase + r0 + r];
    arow[mb] = p.x + (size_t)tok * p.H + 8 * kq;
  }

  f32x4 acc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) acc[mb] = (f32x4){0.f, 0.f, 0.f, 0.f};

  constexpr int U = NMB == 1 ? 4 : 2;
  for (int q0 = w; q0 < nq; q0 += kWaves * U) {
    u32x4 wv[U];
    float2 sv[U];
    u32x4 av[U][2][NMB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = q0 + kWaves * u;
      if (q < nq) {
        wv[u] = load_nt(wt + (size_t)q * kWave);
        sv[u] = sc[(size_t)q * kTileRows];
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb)
            av[u][g][mb] = aval[mb] ? *(const u32x4*)(arow[mb] + kTileK * q + kGroup * g)
                                    : (u32x4){0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = q0 + kWaves * u;
      if (q < nq) {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const bf16x8 b = fp8x8_to_bf16(wv[u][2 * g], wv[u][2 * g + 1]);
          const float s = g ? sv[u].y : sv[u].x;
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) {
            const f32x4 t = mfma16(as_bf16x8(av[u][g][mb]), b);
            acc[mb] += s * t;
          }
        }
      }
    }
  }

  // cross-wave sum in fixed order (wave 0 + 1 + 2 + 3)
  f32x4* red = (f32x4*)L.red;
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) red[(w * 4 + mb) * kWave + lane] = acc[mb];
  __syncthreads();
  if (w < NMB) {
    const int mb = w;
    f32x4 s = red[(0 * 4 + mb) * kWave + lane];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) s += red[(ww * 4 + mb) * kWave + lane];
    // column n < 8 is gate row 8 rb + n, column n + 8 the matching up row
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float g = s[i];
      const float u = __shfl_down(s[i], 8, 16);
      const int r = mb * kMBlock + 4 * kq + i;
      if (n < 8 && r < nrows) {
        const float hv = g / (1.0f + __expf(-g)) * u;
        p.h_scr[(size_t)(sbase + r0 + r) * p.I + 8 * rb + n] = f32_to_bf16(hv);
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Expert down projection: 128 output rows (8 row blocks, 2 per wave, full K =
// I) of one expert for up to 64 of its rows.  Output rows go to o_scr.
// ----------------------------------------------------------------------------
template <int NMB>
__device__ void down_item(const Params& p, int slot, int sbase, int r0, int nrows, int rg) {
  const int w = wave_id(), lane = lane_id();
  const int n = lane & 15, kq = lane >> 4;
  const int nq = p.n_q2;
  const int rb0 = rg * (kDownRows / kTileRows) + 2 * w;

  const uint16_t* arow[NMB];
  bool aval[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    const int r = mb * kMBlock + n;
    aval[mb] = r < nrows;
    arow[mb] = p.h_scr + (size_t)(sbase + r0 + (aval[mb] ? r : 0)) * p.I + 8 * kq;
  }

#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int rb = rb0 + j;
    if (rb >= p.n_rb2) break;
    const size_t blk = (size_t)slot * p.n_rb2 + rb;
    const u32x4* wt = p.w2p + blk * nq * kWave + lane;
    const float2* sc = (const float2*)p.s2p + blk * nq * kTileRows + n;
    f32x4 acc[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) acc[mb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    constexpr int U = NMB == 1 ? 8 : 4;
    for (int q0 = 0; q0 < nq; q0 += U) {
      u32x4 wv[U];
      float2 sv[U];
      u32x4 av[U][2][NMB];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int q = q0 + u;
        if (q < nq) {
          wv[u] = load_nt(wt + (size_t)q * kWave);
          sv[u] = sc[(size_t)q * kTileRows];
#pragma unroll
          for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
              av[u][g][mb] = aval[mb] ? *(const u32x4*)(arow[mb] + kTileK * q + kGroup * g)
                                      : (u32x4){0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int q = q0 + u;
        if (q < nq) {
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const bf16x8 b = fp8x8_to_bf16(wv[u][2 * g], wv[u][2 * g + 1]);
            const float s = g ? sv[u].y : sv[u].x;
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) {
              const f32x4 t = mfma16(as_bf16x8(av[u][g][mb]), b);
              acc[mb] += s * t;
            }
          }
        }
      }
    }
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mb * kMBlock + 4 * kq + i;
        if (r < nrows) p.o_scr[(size_t)(sbase + r0 + r) * p.H + rb * kTileRows + n] = acc[mb][i];
      }
  }
}

// y[t][rg*128 .. +128) = bf16(o_shared + sum_k w_k o_k), in that order.
__device__ void combine_rows(const Params& p, const Lds& L, int ncomb, int rg) {
  const int tid = threadIdx.x;
  const int K = p.K;
  int* ctok = L.comb;                          // [64]
  int* crow = L.comb + kMRange;                // [64][K]
  float* cw = (float*)(L.comb + kMRange + kMRange * kMaxTopK);   // [64][K]
  for (int i = tid; i < ncomb * K; i += kThreads) {
    const int j = i / K, k = i % K;
    const int t = ctok[j];
    const int e = p.topk_idx[t * K + k];
    crow[j * kMaxTopK + k] = pair_row(p, L, t, e);
    cw[j * kMaxTopK + k] = p.topk_w[t * K + k];
  }
  __syncthreads();
  const int c0 = rg * kDownRows;
  const int nc = min(kDownRows, p.H - c0);
  for (int i = tid; i < ncomb * kDownRows; i += kThreads) {
    const int j = i / kDownRows, c = i % kDownRows;
    if (c >= nc) continue;
    const int t = ctok[j];
    float v = p.S ? p.o_scr[(size_t)(p.T * K + t) * p.H + c0 + c] : 0.f;
    for (int k = 0; k < K; ++k)
      v += cw[j * kMaxTopK + k] * p.o_scr[(size_t)crow[j * kMaxTopK + k] * p.H + c0 + c];
    p.y[(size_t)t * p.H + c0 + c] = f32_to_bf16(v);
  }
  __syncthreads();
}

// ----------------------------------------------------------------------------
// The persistent kernel
// ----------------------------------------------------------------------------
template <int NMBMAX>
__global__ void __launch_bounds__(kThreads) moe_decode_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const Lds L = lds_view(p, smem);
  const int tid = threadIdx.x;
  bool placed = false;
  int t_rgu_end = 0, t_total = 0;

  auto ensure_placement = [&]() -> bool {
    if (placed) return true;
    if (!wait_geq(p, p.ctr + kCtrTopkDone, p.n_topk, L.misc + 1)) return false;
    build_placement(p, L);
    const int n_mr = L.misc[2];
    t_rgu_end = p.t_sdn_end + n_mr * p.n_rb13;
    t_total = t_rgu_end + n_mr * p.n_rg;
    placed = true;
    return true;
  };

  // dispatch on the number of 16-row MFMA blocks an item covers
  auto run_gu = [&](int slot, int sbase, int r0, int nrows, int rb, bool shared) {
    const int nmb = (nrows + kMBlock - 1) / kMBlock;
    if (NMBMAX == 1 || nmb <= 1) gu_item<1>(p, L, slot, sbase, r0, nrows, rb, shared);
    else if (nmb == 2) gu_item<NMBMAX >= 2 ? 2 : 1>(p, L, slot, sbase, r0, nrows, rb, shared);
    else if (nmb == 3) gu_item<NMBMAX >= 3 ? 3 : 1>(p, L, slot, sbase, r0, nrows, rb, shared);
    else gu_item<NMBMAX >= 4 ? 4 : 1>(p, L, slot, sbase, r0, nrows, rb, shared);
  };
  auto run_down = [&](int slot, int sbase, int r0, int nrows, int rg) {
    const int nmb = (nrows + kMBlock - 1) / kMBlock;
    if (NMBMAX == 1 || nmb <= 1) down_item<1>(p, slot, sbase, r0, nrows, rg);
    else if (nmb == 2) down_item<NMBMAX >= 2 ? 2 : 1>(p, slot, sbase, r0, nrows, rg);
    else if (nmb == 3) down_item<NMBMAX >= 3 ? 3 : 1>(p, slot, sbase, r0, nrows, rg);
    else down_item<NMBMAX >= 4 ? 4 : 1>(p, slot, sbase, r0, nrows, rg);
  };

  // After a down item: count its rows in for (row, chunk); the last arriver
  // for a (row, chunk) combines it.
  auto arrive_and_combine = [&](int sbase, int r0, int nrows, int rg, bool shared) -> bool {
    __syncthreads();
    if (tid == 0) L.misc[8] = 0;
    __syncthreads();
    if (tid < nrows) {
      const int t = shared ? (r0 + tid) : (int)L.rows[sbase + r0 + tid];
      fence_release_agent();
      const int old = atomic_add_agent(p.pair_done + t * p.n_rg + rg, 1);
      if (old == p.K + p.S - 1) {
        const int j = atomicAdd(L.misc + 8, 1);
        L.comb[j] = t;
      }
    }
    __syncthreads();
    const int ncomb = L.misc[8];
    if (ncomb == 0) return true;
    if (!ensure_placement()) return false;
    if (tid == 0) fence_acquire_agent();
    __syncthreads();
    combine_rows(p, L, ncomb, rg);
    for (int j = tid; j < ncomb; j += kThreads) store_agent(p.pair_done + L.comb[j] * p.n_rg + rg, 0);
    return true;
  };

  bool router_seen = false;
  while (true) {
    if (tid == 0) {
      L.misc[0] = atomic_add_agent(p.ctr + kCtrTicket, 1);
      L.misc[1] = load_agent(p.ctr + kCtrStatus);
    }
    __syncthreads();
    const int tk = L.misc[0];
    const int st = L.misc[1];
    __syncthreads();
    if (st != 0) break;

    if (tk < p.t_router_end) {
      router_item(p, tk);
      publish_done(p.ctr + kCtrRouterDone);
    } else if (tk < p.t_sgu_end) {
      const int i = tk - p.t_router_end;
      const int mr = i / p.n_rb13, rb = i % p.n_rb13;
      const int r0 = mr * kMRange;
      run_gu(p.E, p.T * p.K, r0, min(kMRange, p.T - r0), rb, true);
      publish_done(p.ctr + kCtrHReady + p.E);
    } else if (tk < p.t_topk_end) {
      if (!router_seen) {
        if (!wait_geq(p, p.ctr + kCtrRouterDone, p.n_router, L.misc + 1)) break;
        router_seen = true;
      }
      topk_item(p, tk - p.t_sgu_end);
      publish_done(p.ctr + kCtrTopkDone);
    } else if (tk < p.t_sdn_end) {
      const int i = tk - p.t_topk_end;
      const int mr = i / p.n_rg, rg = i % p.n_rg;
      const int r0 = mr * kMRange;
      const int nrows = min(kMRange, p.T - r0);
      if (!wait_geq(p, p.ctr + kCtrHReady + p.E, p.n_mr_sh * p.n_rb13, L.misc + 1)) break;
      run_down(p.E, p.T * p.K, r0, nrows, rg);
      if (!arrive_and_combine(p.T * p.K, r0, nrows, rg, true)) break;
    } else {
      if (!ensure_placement()) break;
      if (tk >= t_total) break;
      if (tk == p.t_sdn_end) write_placement_debug(p, L);
      if (tk < t_rgu_end) {
        const int i = tk - p.t_sdn_end;
        const int m = i / p.n_rb13, rb = i % p.n_rb13;
        const int e = L.mrlist[m];
        const int r0 = (m - L.nmrb[e]) * kMRange;
        run_gu(e, L.base[e], r0, min(kMRange, L.cnt[e] - r0), rb, false);
        publish_done(p.ctr + kCtrHReady + e);
      } else {
        const int i = tk - t_rgu_end;
        const int m = i / p.n_rg, rg = i % p.n_rg;
        const int e = L.mrlist[m];
        const int r0 = (m - L.nmrb[e]) * kMRange;
        const int nrows = min(kMRange, L.cnt[e] - r0);
        const int need = (L.nmrb[e + 1] - L.nmrb[e]) * p.n_rb13;
        if (!wait_geq(p, p.ctr + kCtrHReady + e, need, L.misc + 1)) break;
        run_down(e, L.base[e], r0, nrows, rg);
        if (!arrive_and_combine(L.base[e], r0, nrows, rg, false)) break;
      }
    }
  }

  // The last workgroup out resets the counters for the next run.
  __syncthreads();
  if (tid == 0) {
    fence_release_agent();
    const int old = atomic_add_agent(p.ctr + kCtrExit, 1);
    if (old == (int)gridDim.x - 1) {
      fence_acquire_agent();
      const bool failed = load_agent(p.ctr + kCtrStatus) != 0;
      store_agent(p.ctr + kCtrTicket, 0);
      store_agent(p.ctr + kCtrRouterDone, 0);
      store_agent(p.ctr + kCtrTopkDone, 0);
      for (int e = 0; e < p.E + p.S; ++e) store_agent(p.ctr + kCtrHReady + e, 0);
      if (failed)
        for (int i = 0; i < p.T * p.n_rg; ++i) store_agent(p.pair_done + i, 0);
      store_agent(p.ctr + kCtrExit, 0);
    }
  }
}

// ----------------------------------------------------------------------------
// Weight re-layout (create time): standard [rows][K] FP8 + [rows][K/32] fp32
// scales -> 1 KiB tiles (see the top of this file).  For the gate/up matrix
// row block rb holds gate rows 8 rb .. 8 rb + 7 then up rows I + 8 rb ..
// I + 8 rb + 7.
// ----------------------------------------------------------------------------
__global__ void pack_kernel(const uint8_t* __restrict__ w, const float* __restrict__ s,
                            u32x4* __restrict__ wp, float* __restrict__ sp, int slots, int rows,
                            int K, int interleave_half) {
  const int nrb = rows / kTileRows, nq = K / kTileK, G = K / kGroup;
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
    if (interleave_half > 0)
      row = n < 8 ? 8 * rb + n : interleave_half + 8 * rb + (n - 8);
    else
      row = kTileRows * rb + n;
    const uint8_t* src = w + ((size_t)slot * rows + row) * K + kTileK * q + 8 * kq;
    const u32x2 a = *(const u32x2*)src;
    const u32x2 b = *(const u32x2*)(src + kGroup);
    wp[i] = (u32x4){a.x, a.y, b.x, b.y};
    if (kq == 0) {
      const float* ss = s + ((size_t)slot * rows + row) * G + 2 * q;
      float* d = sp + (tile * kTileRows + n) * 2;
      d[0] = ss[0];
      d[1] = ss[1];
    }
  }
}

// ----------------------------------------------------------------------------
// Host side
// ----------------------------------------------------------------------------
size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace

struct moe_decode_handle {
  moe_decode_config cfg;
  int device;
  int n_cu;
  float* router_w = nullptr;
  float* router_b = nullptr;
  u32x4* w13p = nullptr;
  float* s13p = nullptr;
  u32x4* w2p = nullptr;
  float* s2p = nullptr;
  float* logits = nullptr;
  int* topk_idx = nullptr;
  float* topk_w = nullptr;
  uint16_t* h_scr = nullptr;
  float* o_scr = nullptr;
  int* ctr = nullptr;
  int* pair_done = nullptr;
  hipStream_t last_stream = nullptr;
  std::mutex mu;
  // occupancy cache, by (kernel variant, LDS bytes)
  int occ_lds[2] = {-1, -1};
  int occ_blocks[2] = {0, 0};
};

namespace {

moe_status check_config(const moe_decode_config* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->flags != 0 || c->deadline_us < 0) return MOE_ERR_INVALID_ARG;
  if (c->max_tokens < 1 || c->hidden < 1 || c->num_experts < 1 || c->top_k < 1 ||
      c->intermediate < 1 || c->num_shared < 0)
    return MOE_ERR_INVALID_ARG;
  if (c->max_tokens > kMaxTokens) return MOE_ERR_UNSUPPORTED;
  if (c->hidden % kTileK != 0 || c->hidden > 16384) return MOE_ERR_UNSUPPORTED;
  if (c->intermediate % kTileK != 0 || c->intermediate > 8192) return MOE_ERR_UNSUPPORTED;
  if (c->num_experts > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (c->top_k > kMaxTopK || c->top_k > c->num_experts) return MOE_ERR_UNSUPPORTED;
  if (c->num_shared > 1) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

Params make_params(const moe_decode_handle* h, int T) {
  const moe_decode_config& c = h->cfg;
  Params p;
  memset(&p, 0, sizeof(p));
  p.T = T;
  p.H = c.hidden;
  p.E = c.num_experts;
  p.K = c.top_k;
  p.S = c.num_shared;
  p.I = c.intermediate;
  p.router_w = h->router_w;
  p.router_b = h->router_b;
  p.w13p = h->w13p;
  p.s13p = h->s13p;
  p.w2p = h->w2p;
  p.s2p = h->s2p;
  p.logits = h->logits;
  p.topk_idx = h->topk_idx;
  p.topk_w = h->topk_w;
  p.h_scr = h->h_scr;
  p.o_scr = h->o_scr;
  p.ctr = h->ctr;
  p.pair_done = h->pair_done;
  const long long dl = c.deadline_us > 0 ? c.deadline_us : 1000000;
  p.deadline_ticks = dl * 100;   // wall clock runs at 100 MHz
  p.n_eb = (p.E + kWaves - 1) / kWaves;
  p.n_rb13 = p.I / 8;
  p.n_q13 = p.H / kTileK;
  p.n_rb2 = p.H / kTileRows;
  p.n_q2 = p.I / kTileK;
  p.n_rg = (p.H + kDownRows - 1) / kDownRows;
  p.nch = (T + 63) / 64;
  p.n_mr_sh = p.S ? (T + kMRange - 1) / kMRange : 0;
  p.n_router = p.n_eb * ((T + kRouterRows - 1) / kRouterRows);
  p.n_topk = (T + kWaves - 1) / kWaves;
  p.t_router_end = p.n_router;
  p.t_sgu_end = p.t_router_end + p.n_mr_sh * p.n_rb13;
  p.t_topk_end = p.t_sgu_end + p.n_topk;
  p.t_sdn_end = p.t_topk_end + p.n_mr_sh * p.n_rg;
  // LDS layout
  const int E = p.E, K = p.K;
  const int max_mr = E + (T * K + kMRange - 1) / kMRange;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 16); return (int)o; };
  p.lds_bm = take((size_t)E * p.nch * 8);
  p.lds_cp = take((size_t)E * p.nch * 4);
  p.lds_cnt = take((size_t)E * 4);
  p.lds_base = take((size_t)E * 4);
  p.lds_nmrb = take((size_t)(E + 1) * 4);
  p.lds_mrlist = take((size_t)max_mr * 4);
  p.lds_rows = take((size_t)T * K * 2);
  const int nmb = T > kMBlock ? 4 : 1;
  p.lds_red = take((size_t)kWaves * 4 * kWave * 16 * (nmb == 1 ? 1 : 1));
  p.lds_comb = take((size_t)(kMRange + 2 * kMRange * kMaxTopK) * 4);
  p.lds_misc = take(16 * 4);
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
  void* ptrs[] = {h->router_w, h->router_b, h->w13p, h->s13p, h->w2p, h->s2p, h->logits,
                  h->topk_idx, h->topk_w, h->h_scr, h->o_scr, h->ctr};
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
  moe_status rc = MOE_OK;
  do {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) { rc = MOE_ERR_HIP; break; }
    h->n_cu = prop.multiProcessorCount;
    const size_t E = cfg->num_experts, S = cfg->num_shared, H = cfg->hidden,
                 I = cfg->intermediate, K = cfg->top_k, Tm = cfg->max_tokens;
    const size_t slots = E + S;
    const size_t n_rg = (H + kDownRows - 1) / kDownRows;
    const size_t scr_rows = Tm * K + Tm * S;
    struct A { void** p; size_t bytes; } allocs[] = {
        {(void**)&h->router_w, E * H * 4},
        {(void**)&h->router_b, w->router_bias ? E * 4 : 0},
        {(void**)&h->w13p, slots * 2 * I * H},
        {(void**)&h->s13p, slots * 2 * I * (H / 32) * 4},
        {(void**)&h->w2p, slots * H * I},
        {(void**)&h->s2p, slots * H * (I / 32) * 4},
        {(void**)&h->logits, Tm * E * 4},
        {(void**)&h->topk_idx, Tm * K * 4},
        {(void**)&h->topk_w, Tm * K * 4},
        {(void**)&h->h_scr, scr_rows * I * 2},
        {(void**)&h->o_scr, scr_rows * H * 4},
        {(void**)&h->ctr, (kCtrHReady + slots + Tm * n_rg) * 4},
    };
    for (auto& a : allocs) {
      if (a.bytes == 0) continue;
      if (hipMalloc(a.p, a.bytes) != hipSuccess) { rc = MOE_ERR_OUT_OF_MEMORY; break; }
    }
    if (rc != MOE_OK) break;
    h->pair_done = h->ctr + kCtrHReady + slots;
    if (hipMemset(h->ctr, 0, (kCtrHReady + slots + Tm * n_rg) * 4) != hipSuccess) { rc = MOE_ERR_HIP; break; }
    if (hipMemcpy(h->router_w, w->router_w, E * H * 4, hipMemcpyDeviceToDevice) != hipSuccess) { rc = MOE_ERR_HIP; break; }
    if (w->router_bias &&
        hipMemcpy(h->router_b, w->router_bias, E * 4, hipMemcpyDeviceToDevice) != hipSuccess) { rc = MOE_ERR_HIP; break; }
    hipLaunchKernelGGL(pack_kernel, dim3(4096), dim3(256), 0, 0, w->w13, w->s13, h->w13p, h->s13p,
                       (int)slots, (int)(2 * I), (int)H, (int)I);
    if (hipGetLastError() != hipSuccess) { rc = MOE_ERR_HIP; break; }
    hipLaunchKernelGGL(pack_kernel, dim3(4096), dim3(256), 0, 0, w->w2, w->s2, h->w2p, h->s2p,
                       (int)slots, (int)H, (int)I, 0);
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

moe_status moe_decode_run(moe_decode_handle* h, const void* x, int32_t T, void* y,
                          const moe_decode_debug* dbg, void* hip_stream) {
  if (!h) return MOE_ERR_INVALID_ARG;
  if (T < 0 || T > h->cfg.max_tokens) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !y) return MOE_ERR_INVALID_ARG;
  if (((uintptr_t)x | (uintptr_t)y) & 15u) return MOE_ERR_INVALID_ARG;
  const size_t bytes = (size_t)T * h->cfg.hidden * 2;
  const uintptr_t xa = (uintptr_t)x, ya = (uintptr_t)y;
  if (xa < ya + bytes && ya < xa + bytes) return MOE_ERR_INVALID_ARG;

  Params p = make_params(h, T);
  p.x = (const uint16_t*)x;
  p.y = (uint16_t*)y;
  if (dbg) {
    p.dbg_idx = dbg->topk_idx;
    p.dbg_w = dbg->topk_w;
    p.dbg_rank = dbg->pair_rank;
    p.dbg_count = dbg->expert_count;
    p.dbg_logits = dbg->logits;
  }
  hipStream_t stream = (hipStream_t)hip_stream;
  std::lock_guard<std::mutex> lock(h->mu);
  int prev = 0;
  HIP_TRY(hipGetDevice(&prev));
  if (prev != h->device) HIP_TRY(hipSetDevice(h->device));
  const int variant = T > kMBlock ? 1 : 0;
  const void* fn = variant ? (const void*)moe_decode_kernel<4> : (const void*)moe_decode_kernel<1>;
  if (h->occ_lds[variant] != p.lds_bytes) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, kThreads, p.lds_bytes) != hipSuccess ||
        nb < 1) {
      if (prev != h->device) (void)hipSetDevice(prev);
      return MOE_ERR_HIP;
    }
    h->occ_lds[variant] = p.lds_bytes;
    h->occ_blocks[variant] = nb;
  }
  const int grid = h->n_cu * h->occ_blocks[variant];
  if (variant)
    hipLaunchKernelGGL(moe_decode_kernel<4>, dim3(grid), dim3(kThreads), p.lds_bytes, stream, p);
  else
    hipLaunchKernelGGL(moe_decode_kernel<1>, dim3(grid), dim3(kThreads), p.lds_bytes, stream, p);
  const hipError_t err = hipGetLastError();
  h->last_stream = stream;
  if (prev != h->device) (void)hipSetDevice(prev);
  return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_decode_check(moe_decode_handle* h) {
  if (!h) return MOE_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(h->mu);
  int prev = 0;
  HIP_TRY(hipGetDevice(&prev));
  if (prev != h->device) HIP_TRY(hipSetDevice(h->device));
  moe_status rc = MOE_OK;
  int status = 0;
  if (hipStreamSynchronize(h->last_stream) != hipSuccess ||
      hipMemcpy(&status, h->ctr + kCtrStatus, 4, hipMemcpyDeviceToHost) != hipSuccess) {
    rc = MOE_ERR_HIP;
  } else if (status != 0) {
    rc = MOE_ERR_TIMEOUT;
    const int zero = 0;
    if (hipMemcpy(h->ctr + kCtrStatus, &zero, 4, hipMemcpyHostToDevice) != hipSuccess) rc = MOE_ERR_HIP;
  }
  if (prev != h->device) (void)hipSetDevice(prev);
  return rc;
}

}  // extern "C"
