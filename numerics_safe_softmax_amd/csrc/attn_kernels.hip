// attn_kernels.hip -- gfx950 (CDNA4) kernels of the stabilised BF16 attention.
//
// Method: web pages on Qiu & Yao, "Why Low-Precision Transformer Training
// Fails: An Analysis on Flash Attention":
//   * itsolotime.com/archives/23922, section "机制解释二": P_bar = exp(S - m),
//     P = P_bar / rowsum(P_bar), O = P V; a repeated row maximum puts exact 1s
//     into P_bar.
//   * same page, section "极简修复方案": count the row maximum's repeats rs;
//     shift by beta*rm (rs > 1, rm > 0), by 0 (rs > 1, rm < 0), else by rm.
//   * 91haoming.cn/news/show-608006, section 三: delta_i = sum_c dO_ic O_ic.
//
// Design (MI355X-first, not a port of the pages' GPU design):
//   * one wave64 owns 32 rows; every dense contraction is a chain of
//     v_mfma_f32_32x32x16_bf16 (bf16 operands, fp32 accumulation);
//   * the score tile is formed with the 32 rows of the wave on the lane axis,
//     so the row max, the duplicate count and the row sum are in-lane
//     reductions plus one exchange between the two 32-lane halves;
//   * the fp32 accumulator layout of one contraction is reused directly as the
//     bf16 B operand of the next (P_bar V, dS K, P^T dO, dS^T Q): the k index
//     of each MFMA is permuted to match, and the other operand is read
//     transposed out of the row-major LDS tile with ds_read_b64_tr_b16;
//   * tiles go global -> LDS directly (buffer_load_dwordx4 ... lds, no
//     staging registers) into an XOR-swizzled row-major layout,
//     double-buffered, one barrier per tile; rows past N are clamped to row
//     N-1 and masked;
//   * the rows a workgroup keeps in registers for the whole loop (Q; Q and
//     dO; K and V) come in the same way, as whole rows, and are read from LDS
//     in the operand layout (loaded straight in that layout, every 16-byte
//     load would touch 32 rows) in the d = 64 forward, the d = 64 dQ pass and
//     the causal d = 64 dK/dV pass; the other kernels load them straight
//     into registers;
//   * a forward tile in which no lane reaches its row's running maximum
//     changes neither the (max, count) pair nor the shift, and skips the
//     count, the merge and the rescale (a wave-uniform test);
//   * all tiles of one (b, h) run on one XCD (its L2 keeps the head's
//     operands) and causal work is ordered heaviest tile first; where a
//     causal grid is resident all at once, the forward and the dQ pass
//     reverse their later dispatch bands (the CUs of the heaviest tiles get
//     the lightest partners) and the dQ and tie-count passes start the
//     lighter tiles later (the heaviest get the start-up bandwidth).
//
// MFMA 32x32x16 lane layout (lane l, half h = l / 32):
//   A (32 x 16): lane l holds row l % 32, k = 8h .. 8h+7
//   B (16 x 32): lane l holds col l % 32, k = 8h .. 8h+7
//   C (32 x 32): element r of lane l is row 8(r/4) + 4h + r%4, col l % 32
// ds_read_b64_tr_b16: within each 16-lane group, lane L supplies an 8-byte
//   address; lane l receives element l%4 of the reads of lanes (l%16)/4 + 4t,
//   t = 0..3.  Reading a 4-row x 16-column block (lane L: row L/4, columns
//   4(L%4)..+3) hands lane l column l%16 of those 4 rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"
#include "pair_schedule.h"

// Tile and occupancy choices (compile-time; the defaults are the variants
// measured fastest on MI355X).
// minimum workgroups per CU in the launch bounds of the dQ and dK/dV passes
#ifndef NSS_DQ_WAVES
#define NSS_DQ_WAVES 2
#endif
#ifndef NSS_DKDV_WAVES
#define NSS_DKDV_WAVES 2
#endif
// keys per key tile of the d = 64 dQ pass
#ifndef NSS_DQ_BN
#define NSS_DQ_BN 64
#endif
// queries per query tile of the d = 64 dK/dV pass
#ifndef NSS_DKDV_BQ
#define NSS_DKDV_BQ 64
#endif
// the d = 64 dK/dV pass reads the next query block's LDS operands while the
// current block's products run (1) or each operand where it is used (0)
#ifndef NSS_DKDV_PF
#define NSS_DKDV_PF 1
#endif

// workgroups per CU the D = 64 forward is compiled for (4: 128 VGPRs)
#ifndef NSS_FWD_WGS
#define NSS_FWD_WGS 4
#endif
// LDS swizzle of the forward kernels' K/V tiles (see Tile): 0 keeps their
// register count down for D = 64
#ifndef NSS_FWD_SWZ
#define NSS_FWD_SWZ 0
#endif
// keys per KV tile of the D = 64 forward (64 or 128)
#ifndef NSS_FWD_BN
#define NSS_FWD_BN 64
#endif

namespace nss {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// LDS swizzle of the forwards' tiles: NSS_FWD_SWZ at D = 64, the
// conflict-free one at D = 128 (its extra address registers still fit three
// workgroups per CU; long_context exact-shift forward 386 -> 379 us, tie
// count -1 %, online forward within noise)
template <int D>
constexpr int kFwdSW = D == 128 ? 1 : NSS_FWD_SWZ;
// Keys per KV tile of the forwards.  D = 128 streams 32-key tiles: two LDS
// stages then take 32 KB and the kernel 164 VGPRs, so three workgroups (3
// waves per SIMD) fit on a CU instead of two with 64-key tiles (long_context
// online forward 341 -> 321 us, plain 339 -> 318, exact final shift 427 ->
// 410 on one box).  The online modes apply the shift tile by tile, so the
// width is part of what they compute (attn_fwd_key_tile reports it).
template <int D>
constexpr int kFwdTile = D == 64 ? NSS_FWD_BN : 32;
// workgroups per CU the forwards are compiled for (launch bounds and the
// resident-grid test of the band order)
template <int D, int BN>
constexpr int kFwdWgs = D == 64 ? NSS_FWD_WGS : (BN == 32 ? 3 : 2);
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// bf16 rounds x to exactly 1.0 (nearest even) iff 1 - 2^-9 <= x <= 1 + 2^-8;
// every P_bar here is at most 1 (plus exp2 rounding), so one compare decides.
constexpr float kBf16OneLow = 0.998046875f;

template <int V>
struct IntC {
  static constexpr int value = V;
};

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine the two 32-lane halves (lane l and lane l ^ 32 hold the same row).
__device__ __forceinline__ float sum32(float v) { return v + __shfl_xor(v, 32); }
__device__ __forceinline__ int sum32i(int v) { return v + __shfl_xor(v, 32); }

// The same exchange through the VALU (gfx950's v_permlane32_swap: the upper
// half of one register trades places with the lower half of another) instead
// of an LDS-crossbar round trip: with a = b = v on entry, every lane ends up
// holding {v(l), v(l ^ 32)} in (a, b), in the same order for every call.
// Written out because this compiler folds the builtin's second result into its
// first; the nops cover the VALU-write -> permlane-read hazard on both sides.
__device__ __forceinline__ void swap_halves(uint32_t v, uint32_t& a, uint32_t& b) {
  a = v;
  b = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}

// Waits for this wave's vector-memory operations (the tile loads into LDS)
// before a barrier.  Written with the builtin rather than inline assembly so
// that the compiler sees the wait: its own wait insertion then knows the
// counter is drained here and does not add a second vmcnt(0) in front of the
// first LDS reads after the next prefetch (gpt2_small dQ pass 29.4 ->
// 28.6 us, sink 72.3 -> 70.7 us, outputs bit-identical).
// s_waitcnt immediate: vmcnt in bits 3:0 and 15:14, expcnt 6:4 (7 = no
// wait), lgkmcnt 11:8 (15 = no wait).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// acc + the sum of eight bf16 values (v_dot2c_f32_bf16 against (1, 1): one
// VALU instruction per pair, the products exact, fp32 accumulation)
__device__ __forceinline__ float add_bf16x8(const bf16x8& p, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int e = 0; e < 8; e += 2) acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p[e], p[e + 1]}, one, acc, false);
  return acc;
}

// eight fp32 accumulator values -> the bf16 B operand of the next contraction.
// SPLIT = 16: k-slice m (0 or 1) takes elements 4m..4m+3 and 8+4m..8+4m+3,
// i.e. score rows 8m + 4h + {0..3} and 16 + 8m + 4h + {0..3} (two row quads 16
// rows apart); SPLIT = 8: elements 8m..8m+7, rows 16m + 4h + {0..3} and
// 16m + 8 + 4h + {0..3}.  The other operand's transposed LDS reads
// (Tile::trans8) follow the same pairing.
template <int SPLIT>
__device__ __forceinline__ bf16x8 pack8(const f32x16& s, int m) {
  static_assert(SPLIT == 8 || SPLIT == 16, "row pairing");
  bf16x8 r;
#pragma unroll
  for (int t = 0; t < 8; t += 2) {
    const int e = SPLIT == 16 ? (t < 4 ? 4 * m : 8 + 4 * m) + (t & 3) : 8 * m + t;
    bf16x2 p = __builtin_convertvector(f32x2{s[e], s[e + 1]}, bf16x2);
    r[t] = p[0];
    r[t + 1] = p[1];
  }
  return r;
}

// ---------------------------------------------------------------------------
// LDS tiles: R rows x D bf16, row-major, rows of D/8 16-byte chunks; chunk c
// of row r sits at chunk c ^ f(r).  The LDS serves 64 four-byte banks (256
// bytes) per cycle; a ds_read_b128 of 64 lanes runs in 16-lane phases, and in
// the row-operand reads (lane l: row l % 32, one chunk) a phase covers 16
// consecutive rows.  f is chosen so those 16 rows fall on distinct banks:
//   D = 64 (two rows per 256 bytes): f = r2 | (r2 ^ r3) << 1 | r1 << 2 is a
//     bijection of (r1, r2, r3), so the eight rows of one parity differ;
//   D = 128 (one row per 256 bytes): f = r2 | (r1 ^ r3) << 1 | r1 << 2 | r0 << 3
//     is a bijection of r mod 16.
// The transposed reads (32 lanes: 4 consecutive rows x 4 chunks) are
// conflict-free too: for D = 64 rows r and r + 2 differ in bit 2 of f, for
// D = 128 rows r .. r + 3 differ in bits 2-3.  f depends on r mod 16 only, so
// the rows r and r + 16 one trans8 call reads (pairing SPLIT = 16) share an
// address pattern.  Because f depends on r3, the two k-slices of a 32-row block
// (8 rows apart) need separate LDS addresses; SW = 0 selects the older
// f = r2 | r0 << 1 | r1 << 2 (distinct banks within 8 rows only: the 16-lane
// row reads take two passes), which depends on r mod 8 only, with the pairing
// SPLIT = 8, for a kernel that cannot spare the registers.
// ---------------------------------------------------------------------------
template <int D, int SW = 1>
struct Tile {
  static constexpr int CPR = D / 8;
  static constexpr int SPLIT = SW == 0 ? 8 : 16;  // row pairing of pack8 / trans8
  __device__ static __forceinline__ int swz(int r) {
    const int r0 = r & 1, r1 = (r >> 1) & 1, r2 = (r >> 2) & 1, r3 = (r >> 3) & 1;
    if constexpr (SW == 0) return r2 | (r0 << 1) | (r1 << 2);
    else if constexpr (D == 64) return r2 | ((r2 ^ r3) << 1) | (r1 << 2);
    else return r2 | ((r1 ^ r3) << 1) | (r1 << 2) | (r0 << 3);
  }
  __device__ static __forceinline__ int chunk(int r, int c) { return r * CPR + (c ^ swz(r)); }
  // 8 bf16 of row r starting at column 8c (an MFMA A/B row operand)
  __device__ static __forceinline__ bf16x8 row8(const uint16_t* t, int r, int c) {
    return as_bf16x8(ld16(t + chunk(r, c) * 8));
  }
  // transposed read: 4 bf16 of rows (the 16-lane block pattern) at column col (multiple of 4)
  __device__ static __forceinline__ u32x2 tr4(const uint16_t* t, int r, int col) {
    const uint16_t* p = t + chunk(r, col >> 3) * 8 + (col & 7);
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    return __builtin_bit_cast(u32x2, v);
  }
  // A operand of X^T for k-slice m of the 32 tile rows from r0 (the pairing of
  // pack8<SPLIT>): for lane l, column 32*cb + l%32, tile rows r0 + 8m + 4h +
  // {0..3} and r0 + 16 + 8m + 4h + {0..3} (SPLIT = 16), or r0 + 16m + 4h +
  // {0..3} and r0 + 16m + 8 + 4h + {0..3} (SPLIT = 8).
  __device__ static __forceinline__ bf16x8 trans8(const uint16_t* t, int r0, int m, int cb, int lane) {
    const int L = lane & 15, h = lane >> 5, G = (lane >> 4) & 1;
    const int r = r0 + (SPLIT == 16 ? 8 : 16) * m + 4 * h + (L >> 2);
    const int col = 32 * cb + 16 * G + 4 * (L & 3);
    const u32x2 a = tr4(t, r, col);
    const u32x2 b = tr4(t, r + SPLIT, col);
    return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
  }
};

// Rows [r0, r0+R) of a bf16 [N][D] matrix straight into a swizzled LDS tile;
// every thread of the 256 issues (R*D/8)/256 16-byte loads.  Rows past N read
// row N-1 (finite data; the kernels mask them).
//
// The loads are buffer_load_dwordx4 ... lds through a resource over the one
// head's matrix (src, N*D*2 bytes: below 2^32 since N < 2^24 and D <= 128, so
// a 32-bit byte offset reaches every row).  The global_load_lds form of the
// same transfer is a FLAT instruction to the compiler, which then cannot
// count LDS reads while a prefetch is in flight and waits for all of them
// (lgkmcnt(0)) before every use; with the buffer form its waits are exact.
// Measured on MI355X, outputs bit-identical: gpt2_small dK/dV 39.7 -> 39.1 us,
// forward 27.4 -> 26.6 us, exact-shift forward 32.0 -> 30.4 us; gpt2_medium
// dK/dV 51.3 -> 48.1 us; sink and long_context backward -3 %.
template <int R, int D, int SW = 1>
__device__ __forceinline__ void tile_to_lds(const uint16_t* __restrict__ src, int r0, int N, uint16_t* tile,
                                            int wu, int lane) {
  constexpr int CPR = D / 8, TOT = R * CPR, PER = TOT / 256;
  static_assert(TOT % 256 == 0, "tile must be a whole number of workgroup loads");
  // dword 3: 32-bit data format, no swizzle, no index stride (raw byte offsets)
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, (int)((uint32_t)N * (uint32_t)D * 2u), 0x00020000);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int P = i * 256 + wu * 64 + lane;
    const int r = P / CPR, p = P % CPR;
    const int c = p ^ Tile<D, SW>::swz(r);
    int gr = r0 + r;
    gr = gr < N ? gr : N - 1;
    // (wu & 3: wu is the wave index 0..3 already, but after readfirstlane the
    // compiler cannot bound it; bounded, it can prove that a prefetch into one
    // stage misses the other and stops waiting for the prefetch before reads
    // of the other stage: dQ pass gpt2_small 29.4 -> 28.9 us, gpt2_medium
    // 41.1 -> 39.3 us; long_context dK/dV 498 -> 490 us; bit-identical)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(tile + (i * 256 + (wu & 3) * 64) * 8), 16,
                                             (int)((uint32_t)(gr * D + c * 8) * 2u), 0, 0, 0);
  }
}

// Dispatch order of a causal grid that is resident all at once: the
// dispatcher places workgroups L, L + 256, L + 512, ... on one CU (seen in
// per-wave traces of the hardware CU id), so the first band of 256 keeps the
// heaviest-first order and every later band runs in reverse, by groups of 8
// so that each head stays on its XCD: the CUs that hold the heaviest causal
// query tiles, whose chains set the forward's span, get the lightest
// partners (gpt2_small online forward 29.3 -> 28.4 us, exact final shift
// 41.7 -> 39.2 us, gpt2_medium within noise; dQ pass with its staggered start
// 31.1 -> 30.4 us).
__device__ __forceinline__ int band_order(int L, int G) {
  constexpr int NCU = 256;
  if (L < NCU) return L;
  const int base = L - L % NCU;
  const int ng = min(NCU, G - base) >> 3, g = (L - base) >> 3;
  return base + 8 * (ng - 1 - g) + (L & 7);
}

// Workgroup L -> (tile rank, head).  Workgroups are dispatched to the 8 XCDs
// round-robin (L % 8); with B*H a multiple of 8 every tile of head bh runs on
// XCD bh % 8.  Rank 0 is dispatched first.
__device__ __forceinline__ void map_block(int L, int BH, int& rank, int& bh) {
  if ((BH & 7) == 0) {
    const int xcd = L & 7, j = L >> 3, hpx = BH >> 3;
    rank = j / hpx;
    bh = (j % hpx) * 8 + xcd;
  } else {
    rank = L / BH;
    bh = L % BH;
  }
}

// The duplicate-max rule in log2-scaled units (base = rm * scale * log2 e).
__device__ __forceinline__ float shifted(float m, int c, float base, int stabilise, float beta) {
  if (stabilise && c > 1) {
    if (m > 0.f) return beta * base;
    if (m < 0.f) return 0.f;
  }
  return base;
}

__device__ __forceinline__ void store_f32x4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

__device__ __forceinline__ void store_bf16x4(uint16_t* p, float a, float b, float c, float d) {
  bf16x2 x = __builtin_convertvector(f32x2{a, b}, bf16x2);
  bf16x2 y = __builtin_convertvector(f32x2{c, d}, bf16x2);
  *reinterpret_cast<u32x2*>(p) = u32x2{__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, y)};
}

// ---------------------------------------------------------------------------
// Forward (and, with TIES_ONLY, the duplicate-max detector alone).
// One workgroup = 128 queries of one (b, h); 4 waves x 32 queries; KV tiles of
// BN keys.  Per tile and wave: S^T = K Q^T, the online (max, count) merge and
// shift, P_bar = exp2(S t - m2), O^T += V^T P_bar^T.
// ---------------------------------------------------------------------------
template <int D, int BN, bool CAUSAL, bool TIES_ONLY>
struct Fwd {
  static constexpr int BM = 128, NKB = BN / 32, NKK = D / 16, NCB = D / 32;
  static constexpr int TILE = BN * D;  // bf16 elements per K or V tile
};

template <int D, int BN, bool CAUSAL, bool TIES_ONLY>
__global__ __launch_bounds__(256, (kFwdWgs<D, BN>)) void fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ O32, float* __restrict__ LSE, int32_t* __restrict__ TIES,
    int32_t* __restrict__ PONE, int32_t* __restrict__ FORMED, float* __restrict__ ROWMAX,
    int BH, int N, float scale, int stabilise, float beta, int nqt) {
  using F = Fwd<D, BN, CAUSAL, TIES_ONLY>;
  constexpr int BM = F::BM, NKB = F::NKB, NKK = F::NKK, NCB = F::NCB, TILE = F::TILE;
  constexpr int NT = TIES_ONLY ? 1 : 2;  // K (and V) per stage
  constexpr int NS = 2;                   // LDS stages: tiles in flight = NS - 1
  constexpr int LOADS = NT * (TILE / 8 / 256);  // 16-byte loads per thread per tile
  __shared__ __attribute__((aligned(16))) uint16_t lds[NS * NT * TILE];
  // QIN: one stage holds the workgroup's Q tile (the d = 64 forward and the
  // tie-count pass with 128-key tiles; the d = 128 forward's 32-key stages are
  // smaller, and its Q rows go straight into registers)
  constexpr bool QIN = NT * TILE >= BM * D;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, h = lane >> 5;
  int rank, bh;
  // the whole grid resident at once
  const bool band = CAUSAL && (BH & 7) == 0 && (int)gridDim.x <= 256 * kFwdWgs<D, BN>;
  map_block(band ? band_order(blockIdx.x, gridDim.x) : (int)blockIdx.x, BH, rank, bh);
  const int qt = CAUSAL ? (nqt - 1 - rank) : rank;
  const size_t head = (size_t)bh * N * D;
  const int q0 = qt * BM, qw = q0 + 32 * wu, qi = qw + li;
  const float t = scale * kLog2e;

  const int kend = CAUSAL ? min(q0 + BM, N) : N;
  const int nkt = (kend + BN - 1) / BN;
  // Staggered start of the duplicate detector (as in the dQ pass, a step of
  // about one rank's Q rows at ~5 TB/s: BH * d / 384 units of 64 clocks):
  // attn_tiecount at gpt2_small 15.2 -> 14.8 us, gpt2_medium 17.8 -> 16.3 us;
  // the online forward, whose tiles also carry the softmax, measured 0.9 us
  // slower with it, and the fused exact-final-shift forward gained nothing
  if (TIES_ONLY && band) {
    const int units = (nqt - 1 - qt) * ((BH * D) / 384);
    for (int i = 0; i < units; i += 8) __builtin_amdgcn_s_sleep(8);
  }
  auto fetch = [&](int kt, int buf) {
    uint16_t* base = lds + buf * NT * TILE;
    tile_to_lds<BN, D, kFwdSW<D>>(K + head, kt * BN, N, base, wu, lane);
    if constexpr (!TIES_ONLY) tile_to_lds<BN, D, kFwdSW<D>>(V + head, kt * BN, N, base + TILE, wu, lane);
  };
  static_assert(NS == 2, "the loop is written for two stages");
  bf16x8 qf[NKK];
  if constexpr (QIN) {
    // Q's rows come in through the second stage (the loop first fills it at
    // tile 1) as whole rows, beside the first KV tile's loads, instead of 32
    // rows per 16-byte load in the operand layout and before them (a Q tile
    // of its own for the 64-key tie-count pass measured slower)
    fetch(0, 0);  // nkt >= 1: the workgroup's first query row is below N
    uint16_t* const qs = lds + NT * TILE;
    tile_to_lds<BM, D, kFwdSW<D>>(Q + head, q0, N, qs, wu, lane);  // rows past N: row N - 1
    wait_vmem();
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[kk] = qi < N ? Tile<D, kFwdSW<D>>::row8(qs, 32 * wu + li, 2 * kk + h) : as_bf16x8(u32x4{0, 0, 0, 0});
  } else {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[kk] = as_bf16x8(qi < N ? ld16(Q + head + (size_t)qi * D + 16 * kk + 8 * h) : u32x4{0, 0, 0, 0});
    wait_vmem();
    fetch(0, 0);
  }

  f32x16 oacc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) oacc[cb] = f32x16{};
  // two row sums: lsum adds the fp32 P_bar (for LSE), lsum_bf the bf16 P_bar
  // that P_bar V consumes (O's normaliser, so that O = sum_j w_j v_j with
  // weights w_j = bf16(P_bar_j) / sum_k bf16(P_bar_k) that sum to 1)
  float m_run = -INFINITY, m2_run = -INFINITY, lsum = 0.f, lsum_bf = 0.f;
  int c_run = 0, ones = 0;
  const bool count_ones = FORMED != nullptr;

  // one KV tile; with two LDS stages the buffer is a compile-time constant
  // (the loop is unrolled by two), so every LDS address is a loop-invariant
  // register plus an immediate offset
  auto tile = [&](const int kt, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    // tile kt has landed once only the later tiles' loads are outstanding
    if (kt + NS - 2 < nkt) wait_vmem_le<LOADS * (NS - 2)>();
    else wait_vmem();
    __syncthreads();
    if (kt + NS - 1 < nkt) fetch(kt + NS - 1, buf ^ 1);
    const uint16_t* Kt = lds + buf * NT * TILE;
    const uint16_t* Vt = Kt + TILE;
    const int k0 = kt * BN;
    const bool active = qw < N && (!CAUSAL || k0 <= qw + 31);
    if (!active) return;

    // LDS operands are read where they are used (no up-front copy of the
    // tile's K and V operands): 128 VGPRs, 4 waves per SIMD at d = 64
    f32x16 s[NKB];
    // scheduling hint: interleave the tile's MFMAs with its other instructions
    // (measured: long_context forward -1 %, the GPT-2 shapes unchanged)
    __builtin_amdgcn_iglp_opt(1);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        s[kb] = mfma(Tile<D, kFwdSW<D>>::row8(Kt, 32 * kb + li, 2 * kk + h), qf[kk], s[kb]);
    if ((CAUSAL && k0 + BN - 1 > qw) || k0 + BN > N) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
          if ((CAUSAL && key > qi) || key >= N) s[kb][r] = -INFINITY;
        }
    }
    // tile (max, count) on the raw fp32 dot products, then the running merge.
    // Each half-row first takes its own (max, count); one exchange then merges
    // the two halves (a half whose max is below the row's adds nothing), so the
    // row count is exactly the number of entries equal to the row max.
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    // A tile in which no lane reaches its row's running maximum changes
    // neither the running (max, count) nor the shift, so alpha is exactly 1:
    // the count, the merge and the rescale are then skipped for the whole wave
    // (a wave-uniform test; outputs bit-identical, the row sum's rescale being
    // one fma with its first add either way).  Rows whose maximum comes early
    // skip most tiles: sink forward 74.5 -> 59.2 us, tie count 27.0 -> 19.3
    // us, long_context forward -2 %; the GPT-2 shapes within noise.
    float alpha = 1.f;
    if (__builtin_amdgcn_ballot_w64(mx >= m_run) != 0) {
      int cnt = 0;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) cnt += (s[kb][r] == mx) ? 1 : 0;
      {
        uint32_t ma, mb, ca, cb;
        swap_halves(__builtin_bit_cast(uint32_t, mx), ma, mb);
        swap_halves((uint32_t)cnt, ca, cb);
        const float fa = __builtin_bit_cast(float, ma), fb = __builtin_bit_cast(float, mb);
        mx = fmaxf(fa, fb);
        cnt = (fa == mx ? (int)ca : 0) + (fb == mx ? (int)cb : 0);
      }
      if (mx == -INFINITY) cnt = 0;
      if (mx > m_run) {
        m_run = mx;
        c_run = cnt;
      } else if (mx == m_run) {
        c_run += cnt;
      }
      if constexpr (!TIES_ONLY) {
        const float base = m_run * t;
        const float m2 = shifted(m_run, c_run, base, stabilise, beta);
        alpha = (m2_run == -INFINITY) ? 0.f : exp2f_fast(m2_run - m2);
        m2_run = m2;
        lsum_bf *= alpha;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) oacc[cb] *= alpha;
      }
    }
    if constexpr (!TIES_ONLY) {
      const float m2 = m2_run;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2f_fast(__builtin_fmaf(s[kb][r], t, -m2));
          s[kb][r] = p;
          lsum = (kb == 0 && r == 0) ? __builtin_fmaf(lsum, alpha, p) : lsum + p;
        }
      if (count_ones) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) ones += (s[kb][r] >= kBf16OneLow) ? 1 : 0;
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 p0 = pack8<Tile<D, kFwdSW<D>>::SPLIT>(s[kb], 0), p1 = pack8<Tile<D, kFwdSW<D>>::SPLIT>(s[kb], 1);
        lsum_bf = add_bf16x8(p1, add_bf16x8(p0, lsum_bf));
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          oacc[cb] = mfma(Tile<D, kFwdSW<D>>::trans8(Vt, 32 * kb, 0, cb, lane), p0, oacc[cb]);
          oacc[cb] = mfma(Tile<D, kFwdSW<D>>::trans8(Vt, 32 * kb, 1, cb, lane), p1, oacc[cb]);
        }
      }
    }
  };
  for (int kt = 0; kt < nkt; kt += 2) {
    tile(kt, IntC<0>{});
    if (kt + 1 < nkt) tile(kt + 1, IntC<1>{});
  }

  if (qw >= N) return;
  const size_t row = (size_t)bh * N + qi;
  if constexpr (TIES_ONLY) {
    if (h == 0 && qi < N) {
      if (TIES) TIES[row] = c_run;
      if (ROWMAX) ROWMAX[row] = scale * m_run;
    }
  } else {
    const float ltot = sum32(lsum);
    const int ones_tot = sum32i(ones);
    const float inv = 1.0f / sum32(lsum_bf);
    if (qi < N) {
      uint16_t* op = O + head + (size_t)qi * D;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          store_bf16x4(op + 32 * cb + 8 * g + 4 * h, oacc[cb][4 * g] * inv, oacc[cb][4 * g + 1] * inv,
                       oacc[cb][4 * g + 2] * inv, oacc[cb][4 * g + 3] * inv);
      if (O32) {  // O before its bf16 rounding (the high-precision delta path)
        float* op32 = O32 + head + (size_t)qi * D;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            store_f32x4(op32 + 32 * cb + 8 * g + 4 * h, oacc[cb][4 * g] * inv, oacc[cb][4 * g + 1] * inv,
                        oacc[cb][4 * g + 2] * inv, oacc[cb][4 * g + 3] * inv);
      }
      if (h == 0) {
        LSE[row] = (m2_run + __builtin_amdgcn_logf(ltot)) * kLn2;
        if (TIES) TIES[row] = c_run;
        if (PONE) {
          const float top = exp2f_fast(m_run * t - m2_run);
          PONE[row] = (__builtin_bit_cast(uint16_t, (__bf16)top) == 0x3F80) ? 1 : 0;
        }
        if (FORMED) FORMED[row] = ones_tot;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The exact-final-shift forward, both passes in one workgroup.  Pass 1
// streams K alone and merges every key tile of each row into its final
// (max, count) (the same merge as fwd_kernel's), from which the rule gives
// the shift m2 (kept in a register; ties and pbar_one are written here).
// Pass 2 streams K and V again and forms every P_bar entry once, with that
// shift, so no entry of a repeated-max row is ever rounded to 1 -- not even
// transiently, as in the online kernel when a duplicate arrives in a later
// tile -- and no rescaling is needed.  One kernel instead of a detector pass
// and a second forward: one start-up and one causal tail fewer, and no shift
// through HBM (gpt2_small 35.3 -> 31.4 us, gpt2_medium 40.6 -> 38.0 us, sink
// 85.5 -> 82.0 us; outputs bit-identical, the merge being exact and
// order-free).
// ---------------------------------------------------------------------------
template <int D, int BN, bool CAUSAL, int BN1>
__global__ __launch_bounds__(256, (kFwdWgs<D, BN>)) void fwd_fixed_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ O32, float* __restrict__ LSE, int32_t* __restrict__ FORMED,
    int32_t* __restrict__ TIES, int32_t* __restrict__ PONE, int BH, int N, float scale, float beta, int nqt) {
  constexpr int BM = 128, NKB = BN / 32, NKK = D / 16, NCB = D / 32, TILE = BN * D;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * 2 * TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, h = lane >> 5;
  int rank, bh;
  // the whole grid resident at once
  const bool band = CAUSAL && (BH & 7) == 0 && (int)gridDim.x <= 256 * kFwdWgs<D, BN>;
  map_block(band ? band_order(blockIdx.x, gridDim.x) : (int)blockIdx.x, BH, rank, bh);
  const int qt = CAUSAL ? (nqt - 1 - rank) : rank;
  const size_t head = (size_t)bh * N * D;
  const int q0 = qt * BM, qw = q0 + 32 * wu, qi = qw + li;
  const size_t row = (size_t)bh * N + qi;
  const float t = scale * kLog2e;

  const int kend = CAUSAL ? min(q0 + BM, N) : N;
  const int nkt = (kend + BN - 1) / BN;
  auto fetch = [&](int kt, int buf) {
    uint16_t* base = lds + buf * 2 * TILE;
    tile_to_lds<BN, D, kFwdSW<D>>(K + head, kt * BN, N, base, wu, lane);
    tile_to_lds<BN, D, kFwdSW<D>>(V + head, kt * BN, N, base + TILE, wu, lane);
  };
  // Q's rows through the second LDS stage as whole rows, as in fwd_kernel
  // pass 1 streams K alone, in tiles of BN1 keys (a stage holds 2 BN keys)
  static_assert(BN1 <= 2 * BN, "a pass-1 key tile fits one stage");
  constexpr int NKB1 = BN1 / 32;
  const int nkt1 = (kend + BN1 - 1) / BN1;
  auto fetch_k = [&](int kt, int buf) {
    tile_to_lds<BN1, D, kFwdSW<D>>(K + head, kt * BN1, N, lds + buf * 2 * TILE, wu, lane);
  };
  fetch_k(0, 0);
  bf16x8 qf[NKK];
  if constexpr (2 * TILE >= BM * D) {
    uint16_t* const qs = lds + 2 * TILE;
    tile_to_lds<BM, D, kFwdSW<D>>(Q + head, q0, N, qs, wu, lane);  // rows past N: row N - 1
    wait_vmem();
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[kk] = qi < N ? Tile<D, kFwdSW<D>>::row8(qs, 32 * wu + li, 2 * kk + h) : as_bf16x8(u32x4{0, 0, 0, 0});
  } else {
    // the second stage is smaller than the Q tile (D = 128, 32-key tiles):
    // the rows go straight into registers
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[kk] = as_bf16x8(qi < N ? ld16(Q + head + (size_t)qi * D + 16 * kk + 8 * h) : u32x4{0, 0, 0, 0});
  }
  // pass 1: the whole row's (max, count) over the key tiles, then the rule's
  // shift from it (the same merge as fwd_kernel's)
  float m_run = -INFINITY;
  int c_run = 0;
  auto tile1 = [&](const int kt, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    wait_vmem();
    __syncthreads();
    if (kt + 1 < nkt1) fetch_k(kt + 1, buf ^ 1);
    const uint16_t* Kt = lds + buf * 2 * TILE;
    const int k0 = kt * BN1;
    const bool active = qw < N && (!CAUSAL || k0 <= qw + 31);
    if (!active) return;
    f32x16 s[NKB1];
    __builtin_amdgcn_iglp_opt(1);
#pragma unroll
    for (int kb = 0; kb < NKB1; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int kb = 0; kb < NKB1; ++kb)
        s[kb] = mfma(Tile<D, kFwdSW<D>>::row8(Kt, 32 * kb + li, 2 * kk + h), qf[kk], s[kb]);
    if ((CAUSAL && k0 + BN1 - 1 > qw) || k0 + BN1 > N) {
#pragma unroll
      for (int kb = 0; kb < NKB1; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
          if ((CAUSAL && key > qi) || key >= N) s[kb][r] = -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < NKB1; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    // (as in fwd_kernel: a tile below every lane's running maximum changes nothing)
    if (__builtin_amdgcn_ballot_w64(mx >= m_run) == 0) return;
    int cnt = 0;
#pragma unroll
    for (int kb = 0; kb < NKB1; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) cnt += (s[kb][r] == mx) ? 1 : 0;
    {
      uint32_t ma, mb, ca, cb;
      swap_halves(__builtin_bit_cast(uint32_t, mx), ma, mb);
      swap_halves((uint32_t)cnt, ca, cb);
      const float fa = __builtin_bit_cast(float, ma), fb = __builtin_bit_cast(float, mb);
      mx = fmaxf(fa, fb);
      cnt = (fa == mx ? (int)ca : 0) + (fb == mx ? (int)cb : 0);
    }
    if (mx == -INFINITY) cnt = 0;
    if (mx > m_run) {
      m_run = mx;
      c_run = cnt;
    } else if (mx == m_run) {
      c_run += cnt;
    }
  };
  for (int kt = 0; kt < nkt1; kt += 2) {
    tile1(kt, IntC<0>{});
    if (kt + 1 < nkt1) tile1(kt + 1, IntC<1>{});
  }
  const float base = m_run * t;
  const float m2 = qi < N ? shifted(m_run, c_run, base, 1, beta) : 0.f;
  if (h == 0 && qi < N) {
    if (TIES) TIES[row] = c_run;
    if (PONE) PONE[row] = (__builtin_bit_cast(uint16_t, (__bf16)exp2f_fast(base - m2)) == 0x3F80) ? 1 : 0;
  }
  __syncthreads();  // every wave is done with the last key tile: pass 2 reloads the stages
  fetch(0, 0);

  f32x16 oacc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) oacc[cb] = f32x16{};
  float lsum = 0.f, lsum_bf = 0.f;  // fp32 P_bar (LSE) and bf16 P_bar (O), as in fwd_kernel
  int ones = 0;
  const bool count_ones = FORMED != nullptr;

  // one KV tile (LDS buffer a compile-time constant, as in fwd_kernel)
  auto tile = [&](const int kt, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    wait_vmem();
    __syncthreads();
    if (kt + 1 < nkt) fetch(kt + 1, buf ^ 1);
    const uint16_t* Kt = lds + buf * 2 * TILE;
    const uint16_t* Vt = Kt + TILE;
    const int k0 = kt * BN;
    const bool active = qw < N && (!CAUSAL || k0 <= qw + 31);
    if (!active) return;

    f32x16 s[NKB];
    // scheduling hint: interleave the tile's MFMAs with its other instructions
    // (measured: long_context forward -1 %, the GPT-2 shapes unchanged)
    __builtin_amdgcn_iglp_opt(1);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        s[kb] = mfma(Tile<D, kFwdSW<D>>::row8(Kt, 32 * kb + li, 2 * kk + h), qf[kk], s[kb]);
    if ((CAUSAL && k0 + BN - 1 > qw) || k0 + BN > N) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
          if ((CAUSAL && key > qi) || key >= N) s[kb][r] = -INFINITY;
        }
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f_fast(__builtin_fmaf(s[kb][r], t, -m2));
        s[kb][r] = p;
        lsum += p;
      }
    if (count_ones) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) ones += (s[kb][r] >= kBf16OneLow) ? 1 : 0;
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const bf16x8 p0 = pack8<Tile<D, kFwdSW<D>>::SPLIT>(s[kb], 0), p1 = pack8<Tile<D, kFwdSW<D>>::SPLIT>(s[kb], 1);
      lsum_bf = add_bf16x8(p1, add_bf16x8(p0, lsum_bf));
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        oacc[cb] = mfma(Tile<D, kFwdSW<D>>::trans8(Vt, 32 * kb, 0, cb, lane), p0, oacc[cb]);
        oacc[cb] = mfma(Tile<D, kFwdSW<D>>::trans8(Vt, 32 * kb, 1, cb, lane), p1, oacc[cb]);
      }
    }
  };
  for (int kt = 0; kt < nkt; kt += 2) {
    tile(kt, IntC<0>{});
    if (kt + 1 < nkt) tile(kt + 1, IntC<1>{});
  }

  if (qw >= N) return;
  const float ltot = sum32(lsum);
  const int ones_tot = sum32i(ones);
  const float inv = 1.0f / sum32(lsum_bf);
  if (qi >= N) return;
  uint16_t* op = O + head + (size_t)qi * D;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      store_bf16x4(op + 32 * cb + 8 * g + 4 * h, oacc[cb][4 * g] * inv, oacc[cb][4 * g + 1] * inv,
                   oacc[cb][4 * g + 2] * inv, oacc[cb][4 * g + 3] * inv);
  if (O32) {
    float* op32 = O32 + head + (size_t)qi * D;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store_f32x4(op32 + 32 * cb + 8 * g + 4 * h, oacc[cb][4 * g] * inv, oacc[cb][4 * g + 1] * inv,
                    oacc[cb][4 * g + 2] * inv, oacc[cb][4 * g + 3] * inv);
  }
  if (h == 0) {
    LSE[row] = (m2 + __builtin_amdgcn_logf(ltot)) * kLn2;
    if (FORMED) FORMED[row] = ones_tot;
  }
}

// ---------------------------------------------------------------------------
// Backward, query side: delta_i = sum_c dO_ic O_ic, then for each KV tile
// S^T = K Q^T, P = exp2(S t - lse2), dP^T = V dO^T, dS = P (dP - delta),
// dQ^T += K^T dS^T.  One workgroup = 128 queries; KV tiles of BN keys.
// ---------------------------------------------------------------------------
template <int D, int BN, bool CAUSAL, bool O32>
__global__ __launch_bounds__(256, NSS_DQ_WAVES) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const void* __restrict__ Og, const uint16_t* __restrict__ dO, const float* __restrict__ LSE,
    uint16_t* __restrict__ dQ, float* __restrict__ DELTA, int BH, int N, float scale, int nqt) {
  constexpr int BM = 128, NKB = BN / 32, NKK = D / 16, NCB = D / 32, TILE = BN * D;
  // STAGE: the workgroup's Q and dO rows come in through LDS (48 KB per
  // workgroup at d = 64, still three per CU); at d = 128 the two stages alone
  // take 64 KB and the rows are loaded straight into registers
  constexpr bool STAGE = D == 64 && !O32;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * 2 * TILE];
  __shared__ __attribute__((aligned(16))) uint16_t qst[STAGE ? BM * D : 8];
  __shared__ float dlt[STAGE ? BM : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, h = lane >> 5;
  int rank, bh;
  // the whole grid resident at once: 3 workgroups per CU at d = 64, 2 at d = 128
  const bool resident = CAUSAL && (int)gridDim.x <= (D == 64 ? 768 : 512);
  map_block(resident && (BH & 7) == 0 ? band_order(blockIdx.x, gridDim.x) : (int)blockIdx.x, BH, rank, bh);
  const int qt = CAUSAL ? (nqt - 1 - rank) : rank;
  const size_t head = (size_t)bh * N * D;
  const int q0 = qt * BM, qw = q0 + 32 * wu, qi = qw + li;
  const float t = scale * kLog2e;

  const int kend = CAUSAL ? min(q0 + BM, N) : N;
  const int nkt = (kend + BN - 1) / BN;
  // Staggered start (causal, the whole grid resident at once): every
  // workgroup loads its rows at the same time, and the first tile is ready
  // only when most of those bytes have arrived.  The workgroups of lighter
  // query tiles therefore wait before their first loads, one step per rank
  // below the heaviest, a step of about the time one rank's rows take to load
  // (BH * 128 rows * 6d bytes of Q, dO and O at ~5 TB/s: BH * d / 128 units of
  // s_sleep's 64 clocks), so that the heaviest tiles, whose chains set the
  // pass's span, get the start-up bandwidth (gpt2_small dQ 30.9 -> 29.9 us;
  // steps of 2/3 and 4/3 of that gained less, twice it lost).
  if (resident) {
    const int units = (nqt - 1 - qt) * ((BH * D) >> 7);
    for (int i = 0; i < units; i += 8) __builtin_amdgcn_s_sleep(8);
  }
  auto fetch = [&](int kt, int buf) {
    uint16_t* base = lds + buf * 2 * TILE;
    tile_to_lds<BN, D>(K + head, kt * BN, N, base, wu, lane);
    tile_to_lds<BN, D>(V + head, kt * BN, N, base + TILE, wu, lane);
  };
  fetch(0, 0);

  bf16x8 qf[NKK], gf[NKK];
  float dl = 0.f;
  const u32x4 z{0, 0, 0, 0};
  if constexpr (STAGE) {
    // The operand layout puts 32 rows in every 16-byte load (lane l: row l %
    // 32), so a prologue loading Q, dO and O that way moves 32-byte pieces of
    // 96 rows per instruction.  Instead Q and dO go to LDS as whole rows (the
    // key tiles' loads: eight lanes per 128-byte row), into a tile of their
    // own and into the second key stage, which the loop first fills at its
    // first tile; O is loaded as whole rows too, for delta only (lane l: row
    // 8i + l/8 of the wave's 32, columns 8(l%8)..+7).
    uint16_t* const dst = lds + 2 * TILE;
    tile_to_lds<BM, D>(Q + head, q0, N, qst, wu, lane);
    tile_to_lds<BM, D>(dO + head, q0, N, dst, wu, lane);
    const uint16_t* O = static_cast<const uint16_t*>(Og);
    bf16x8 oc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = qw + 8 * i + (lane >> 3);
      oc[i] = as_bf16x8(r < N ? ld16(O + head + (size_t)r * D + 8 * (lane & 7)) : z);
    }
    wait_vmem();
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      qf[kk] = Tile<D>::row8(qst, 32 * wu + li, 2 * kk + h);
      gf[kk] = Tile<D>::row8(dst, 32 * wu + li, 2 * kk + h);
    }
    // delta_r = sum_c dO_rc O_rc: eight products per lane, then the sum over
    // the row's eight lanes, handed to the row's lane through LDS
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 32 * wu + 8 * i + (lane >> 3);
      const bf16x8 g = Tile<D>::row8(dst, r, lane & 7);
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) p = __builtin_fmaf((float)g[e], (float)oc[i][e], p);
      p += __shfl_xor(p, 1);
      p += __shfl_xor(p, 2);
      p += __shfl_xor(p, 4);
      if ((lane & 7) == 0) dlt[r] = p;
    }
    dl = dlt[32 * wu + li];
    if (qi >= N) {  // rows past N: the loads above read row N - 1 there
      dl = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) qf[kk] = gf[kk] = as_bf16x8(z);
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const size_t off = head + (size_t)qi * D + 16 * kk + 8 * h;
      qf[kk] = as_bf16x8(qi < N ? ld16(Q + off) : z);
      gf[kk] = as_bf16x8(qi < N ? ld16(dO + off) : z);
      if constexpr (O32) {  // delta from O before its bf16 rounding
        const float* o32 = static_cast<const float*>(Og) + off;
        const f32x4 a = qi < N ? *reinterpret_cast<const f32x4*>(o32) : f32x4{};
        const f32x4 b = qi < N ? *reinterpret_cast<const f32x4*>(o32 + 4) : f32x4{};
#pragma unroll
        for (int e = 0; e < 4; ++e) dl += (float)gf[kk][e] * a[e] + (float)gf[kk][e + 4] * b[e];
      } else {
        const bf16x8 of = as_bf16x8(qi < N ? ld16(static_cast<const uint16_t*>(Og) + off) : z);
#pragma unroll
        for (int e = 0; e < 8; ++e) dl += (float)gf[kk][e] * (float)of[e];
      }
    }
    dl = sum32(dl);
  }
  const float lse2 = qi < N ? LSE[(size_t)bh * N + qi] * kLog2e : 0.f;
  if (h == 0 && qi < N) DELTA[(size_t)bh * N + qi] = dl;

  f32x16 dqa[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) dqa[cb] = f32x16{};

  // dP accumulates onto -delta (one value per query, i.e. per lane), so
  // dP - delta comes out of the products
  f32x16 negd;
#pragma unroll
  for (int r = 0; r < 16; ++r) negd[r] = -dl;

  // one key tile; the LDS buffer is a compile-time constant so that every LDS
  // address is a loop-invariant register plus an immediate offset
  auto tile = [&](const int kt, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    wait_vmem();
    __syncthreads();
    if (kt + 1 < nkt) fetch(kt + 1, buf ^ 1);
    const uint16_t* Kt = lds + buf * 2 * TILE;
    const uint16_t* Vt = Kt + TILE;
    const int k0 = kt * BN;
    const bool active = qw < N && (!CAUSAL || k0 <= qw + 31);
    if (!active) return;

    // one 32-key block at a time: S, dP, dS, then dQ (halves the live score
    // registers)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x16 s = f32x16{}, dp = negd;
      // scheduling hint for the block's MFMA / LDS / vector interleave at
      // d = 64 (measured: gpt2_medium dQ 38.7 -> 37.8 us, sink 70.3 -> 69.8
      // us, gpt2_small within noise; long_context, d = 128, 374 -> 377 us, so
      // not there; outputs bit-identical)
      if constexpr (D == 64) __builtin_amdgcn_iglp_opt(0);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        s = mfma(Tile<D>::row8(Kt, 32 * kb + li, 2 * kk + h), qf[kk], s);
        dp = mfma(Tile<D>::row8(Vt, 32 * kb + li, 2 * kk + h), gf[kk], dp);
      }
      if ((CAUSAL && k0 + 32 * kb + 31 > qw) || k0 + 32 * kb + 32 > N) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
          if ((CAUSAL && key > qi) || key >= N) s[r] = -INFINITY;
        }
      }
      // d = 64: the first column block's transposed K operands are read ahead
      // of the vector work, so that their latency hides behind it (the
      // scheduling barrier keeps the compiler from sinking them back to their
      // products; 168 VGPRs, still 3 waves per SIMD): gpt2_small dQ 28.9 ->
      // 28.0 us, gpt2_medium 37.6 -> 37.4, sink 70.2 -> 69.8; bit-identical
      // (at d = 128 long_context measured 364 -> 373 us, so not there)
      constexpr bool RA = (D == 64);
      bf16x8 tk0{}, tk1{};
      if constexpr (RA) {
        tk0 = Tile<D>::trans8(Kt, 32 * kb, 0, 0, lane);
        tk1 = Tile<D>::trans8(Kt, 32 * kb, 1, 0, lane);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f_fast(__builtin_fmaf(s[r], t, -lse2));
        s[r] = p * dp[r];
      }
      const bf16x8 d0 = pack8<Tile<D>::SPLIT>(s, 0), d1 = pack8<Tile<D>::SPLIT>(s, 1);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        dqa[cb] = mfma(RA && cb == 0 ? tk0 : Tile<D>::trans8(Kt, 32 * kb, 0, cb, lane), d0, dqa[cb]);
        dqa[cb] = mfma(RA && cb == 0 ? tk1 : Tile<D>::trans8(Kt, 32 * kb, 1, cb, lane), d1, dqa[cb]);
      }
    }
  };
  for (int kt = 0; kt < nkt; kt += 2) {
    tile(kt, IntC<0>{});
    if (kt + 1 < nkt) tile(kt + 1, IntC<1>{});
  }

  if (qi >= N) return;
  uint16_t* qp = dQ + head + (size_t)qi * D;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      store_bf16x4(qp + 32 * cb + 8 * g + 4 * h, dqa[cb][4 * g] * scale, dqa[cb][4 * g + 1] * scale,
                   dqa[cb][4 * g + 2] * scale, dqa[cb][4 * g + 3] * scale);
}

// ---------------------------------------------------------------------------
// Backward, key side: one workgroup = 128 keys (4 waves x 32); query tiles of
// BQ rows.  Per tile: S = Q K^T (keys on the lane axis), P = exp2(S t - lse2),
// dP = dO V^T, dS = P (dP - delta), dV^T += dO^T P, dK^T += Q^T dS.
//
// Causal grids with more key tiles per XCD than its CUs hold at once (two
// workgroups per CU) are packed into one such round: with `single` >= 0, the
// first `single` workgroups of an XCD take its heaviest key tiles alone and
// the others a heavy + light pair each (the tiles single + p and nloc - 1 - p),
// and the launcher places the pairs so that the CUs' work evens out and the
// two workgroups of a CU share a head where they can (gpt2_small dK/dV 39.9
// -> 39.5 us for the pairing, then 38.6 -> 37.6 us for the placement, two
// boxes; gpt2_medium 49.2 -> 48.2 us; sink and long_context within noise;
// outputs bit-identical).  Each key tile is computed exactly as by a
// workgroup of its own.
// ---------------------------------------------------------------------------

template <int D, int BQ, bool CAUSAL>
__global__ __launch_bounds__(256, NSS_DKDV_WAVES) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ DELTA,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int BH, int N, float scale, int nkt, int single,
    PairOrder ord) {
  constexpr int BK = 128, NQB = BQ / 32, NKK = D / 16, NCB = D / 32, TILE = BQ * D;
  // d = 128: the workgroup's V rows sit in LDS (32 KB) and are read as the dP
  // products' B operand where used, instead of 32 VGPRs per lane: the kernel
  // then fits 2 waves per SIMD (long_context dK/dV 709 -> 522 us)
  constexpr bool VL = (D == 128);
  __shared__ __attribute__((aligned(16))) uint16_t vtile[VL ? BK * D : 8];
  // d = 64: each block's LDS operands are read ahead of their use, and each
  // LDS stage is a variable of its own: reading one stage then cannot alias
  // the global->LDS loads into the other, so the compiler does not wait for
  // the prefetch of the next tile before the first LDS reads of this one
  // (at d = 128 the single buffer measured faster)
  constexpr bool PF = !VL && NSS_DKDV_PF;
  __shared__ __attribute__((aligned(16))) uint16_t ldsA[PF ? 2 * TILE : 4 * TILE];
  __shared__ __attribute__((aligned(16))) uint16_t ldsB[PF ? 2 * TILE : 8];
  uint16_t* const lds0 = ldsA;
  uint16_t* const lds1 = PF ? ldsB : ldsA + 2 * TILE;
  __shared__ __attribute__((aligned(16))) float rowv[2][2][BQ];  // [buf][lse2, delta][row]
  // d = 64, causal: the workgroup's K and V rows come in through LDS as whole
  // rows (a 32 KB tile; two workgroups per CU leave room) rather than 32 rows
  // per 16-byte load in the operand layout (gpt2_small dK/dV 41.7 -> 39.6 us;
  // non-causal sink measured 100 -> 103 us, so that case loads as before)
  constexpr bool STAGE = !VL && CAUSAL;
  __shared__ __attribute__((aligned(16))) uint16_t kvst[STAGE ? 2 * BK * D : 8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, h = lane >> 5;
  // the workgroup's key tiles (linear indices as map_block takes them; index
  // L runs on XCD L % 8, so both tiles of a pair belong to this XCD)
  int item0 = blockIdx.x, item1 = -1;
  if (CAUSAL && single >= 0) {
    const int jl = blockIdx.x >> 3, nloc = (BH >> 3) * nkt, x = blockIdx.x & 7;
    if (jl >= single) {
      // one round (nloc <= 128): the pair the launcher placed on this slot
      const int pr = nloc <= 128 ? (int)ord.p[jl - single] : jl - single;
      item0 = 8 * (single + pr) + x;
      item1 = 8 * (nloc - 1 - pr) + x;
    }
  }
  auto body = [&](const int L) {
  int rank, bh;
  map_block(L, BH, rank, bh);
  const int kt = rank;  // causal: the first key tiles see the most queries
  const size_t head = (size_t)bh * N * D;
  const size_t hrow = (size_t)bh * N;
  const int k0 = kt * BK, kw = k0 + 32 * wu, kj = kw + li;
  const float t = scale * kLog2e;

  const int qstart = CAUSAL ? (k0 / BQ) : 0;
  const int nqt = (N + BQ - 1) / BQ;
  float rl = 0.f, rd = 0.f;
  auto fetch = [&](int qt, uint16_t* base) {
    tile_to_lds<BQ, D>(Q + head, qt * BQ, N, base, wu, lane);
    tile_to_lds<BQ, D>(dO + head, qt * BQ, N, base + TILE, wu, lane);
    if (tid < BQ) {
      int r = qt * BQ + tid;
      r = r < N ? r : N - 1;
      rl = LSE[hrow + r];
      rd = DELTA[hrow + r];
    }
  };
  auto commit_rows = [&](int buf) {
    if (tid < BQ) {
      rowv[buf][0][tid] = rl * kLog2e;
      rowv[buf][1][tid] = -rd;  // -delta: the initial value of the dP accumulator
    }
  };
  if constexpr (VL) tile_to_lds<BK, D>(V + head, k0, N, vtile, wu, lane);  // rows past N: row N-1, unused
  if constexpr (STAGE) {
    tile_to_lds<BK, D>(K + head, k0, N, kvst, wu, lane);  // rows past N: row N-1, zeroed below
    tile_to_lds<BK, D>(V + head, k0, N, kvst + BK * D, wu, lane);
  }
  fetch(qstart, lds0);

  bf16x8 kf[NKK], vf[VL ? 1 : NKK];
  const u32x4 z{0, 0, 0, 0};
  if constexpr (!STAGE) {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const size_t off = head + (size_t)kj * D + 16 * kk + 8 * h;
      kf[kk] = as_bf16x8(kj < N ? ld16(K + off) : z);
      if constexpr (!VL) vf[kk] = as_bf16x8(kj < N ? ld16(V + off) : z);
    }
  }
  f32x16 dka[NCB], dva[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    dka[cb] = f32x16{};
    dva[cb] = f32x16{};
  }
  wait_vmem();
  if constexpr (STAGE) {
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      kf[kk] = kj < N ? Tile<D>::row8(kvst, 32 * wu + li, 2 * kk + h) : as_bf16x8(z);
      vf[kk] = kj < N ? Tile<D>::row8(kvst + BK * D, 32 * wu + li, 2 * kk + h) : as_bf16x8(z);
    }
  }
  commit_rows(0);

  // one query tile; the LDS buffer is a compile-time constant so that every
  // LDS address is a loop-invariant register plus an immediate offset
  auto tile = [&](const int qt, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    wait_vmem();
    __syncthreads();
    if (qt + 1 < nqt) fetch(qt + 1, buf ? lds0 : lds1);
    const uint16_t* Qt = buf ? lds1 : lds0;
    const uint16_t* Gt = Qt + TILE;
    const int r0 = qt * BQ;
    const bool active = kw < N && (!CAUSAL || r0 + BQ - 1 >= kw);
    if (active) {
      // one 32-query block at a time: S, dP, then P, dS, then dV, dK (halves
      // the live score registers)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        if constexpr (PF) {
          // every LDS operand of the block is read ahead of its use: the S
          // and dP operands before their products, and the dV / dK operands
          // right behind those products, so that their latency hides behind
          // the products and the vector work instead of stalling each
          // product pair
          // scheduling hint for the block's MFMA / LDS / vector interleave
          // (measured: sink dK/dV -4 %, gpt2_medium -1 %, gpt2_small unchanged)
          __builtin_amdgcn_iglp_opt(0);
          f32x4 d4[4], l4[4];
          bf16x8 qa[NKK], ga[NKK];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            d4[g] = *reinterpret_cast<const f32x4*>(&rowv[buf][1][32 * qb + 8 * g + 4 * h]);
            l4[g] = *reinterpret_cast<const f32x4*>(&rowv[buf][0][32 * qb + 8 * g + 4 * h]);
          }
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk) {
            qa[kk] = Tile<D>::row8(Qt, 32 * qb + li, 2 * kk + h);
            ga[kk] = Tile<D>::row8(Gt, 32 * qb + li, 2 * kk + h);
          }
          // dP accumulates onto -delta, so dP - delta comes out of the products
          f32x16 s = f32x16{}, dp;
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) dp[4 * g + jj] = d4[g][jj];
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk) {
            s = mfma(qa[kk], kf[kk], s);
            dp = mfma(ga[kk], vf[kk], dp);
          }
          bf16x8 tg[NCB][2], tq[NCB][2];
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int m = 0; m < 2; ++m) {
              tg[cb][m] = Tile<D>::trans8(Gt, 32 * qb, m, cb, lane);
              tq[cb][m] = Tile<D>::trans8(Qt, 32 * qb, m, cb, lane);
            }
          __builtin_amdgcn_sched_barrier(0);
          if ((CAUSAL && r0 + 32 * qb < kw + 31) || r0 + 32 * qb + 32 > N) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int qrow = r0 + 32 * qb + 8 * (r >> 2) + 4 * h + (r & 3);
              if ((CAUSAL && qrow < kj) || qrow >= N) s[r] = -INFINITY;
            }
          }
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const int r = 4 * g + jj;
              const float p = exp2f_fast(__builtin_fmaf(s[r], t, -l4[g][jj]));
              s[r] = p;
              dp[r] = p * dp[r];
            }
          const bf16x8 p0 = pack8<Tile<D>::SPLIT>(s, 0), p1 = pack8<Tile<D>::SPLIT>(s, 1);
          const bf16x8 d0 = pack8<Tile<D>::SPLIT>(dp, 0), d1 = pack8<Tile<D>::SPLIT>(dp, 1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            dva[cb] = mfma(tg[cb][0], p0, dva[cb]);
            dva[cb] = mfma(tg[cb][1], p1, dva[cb]);
            dka[cb] = mfma(tq[cb][0], d0, dka[cb]);
            dka[cb] = mfma(tq[cb][1], d1, dka[cb]);
          }
          continue;
        }
        // dP accumulates onto -delta, so dP - delta comes out of the products
        f32x16 s = f32x16{}, dp;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&rowv[buf][1][32 * qb + 8 * g + 4 * h]);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) dp[4 * g + jj] = d4[jj];
        }
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          s = mfma(Tile<D>::row8(Qt, 32 * qb + li, 2 * kk + h), kf[kk], s);
          if constexpr (VL)
            dp = mfma(Tile<D>::row8(Gt, 32 * qb + li, 2 * kk + h), Tile<D>::row8(vtile, 32 * wu + li, 2 * kk + h),
                      dp);
          else
            dp = mfma(Tile<D>::row8(Gt, 32 * qb + li, 2 * kk + h), vf[kk], dp);
        }
        if ((CAUSAL && r0 + 32 * qb < kw + 31) || r0 + 32 * qb + 32 > N) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qrow = r0 + 32 * qb + 8 * (r >> 2) + 4 * h + (r & 3);
            if ((CAUSAL && qrow < kj) || qrow >= N) s[r] = -INFINITY;
          }
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&rowv[buf][0][32 * qb + 8 * g + 4 * h]);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int r = 4 * g + jj;
            const float p = exp2f_fast(__builtin_fmaf(s[r], t, -l4[jj]));
            s[r] = p;
            dp[r] = p * dp[r];
          }
        }
        const bf16x8 p0 = pack8<Tile<D>::SPLIT>(s, 0), p1 = pack8<Tile<D>::SPLIT>(s, 1);
        const bf16x8 d0 = pack8<Tile<D>::SPLIT>(dp, 0), d1 = pack8<Tile<D>::SPLIT>(dp, 1);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          dva[cb] = mfma(Tile<D>::trans8(Gt, 32 * qb, 0, cb, lane), p0, dva[cb]);
          dva[cb] = mfma(Tile<D>::trans8(Gt, 32 * qb, 1, cb, lane), p1, dva[cb]);
          dka[cb] = mfma(Tile<D>::trans8(Qt, 32 * qb, 0, cb, lane), d0, dka[cb]);
          dka[cb] = mfma(Tile<D>::trans8(Qt, 32 * qb, 1, cb, lane), d1, dka[cb]);
        }
      }
    }
    if (qt + 1 < nqt) {
      wait_vmem();
      commit_rows(buf ^ 1);
    }
  };
  for (int qt = qstart; qt < nqt; qt += 2) {
    tile(qt, IntC<0>{});
    if (qt + 1 < nqt) tile(qt + 1, IntC<1>{});
  }

  if (kj >= N) return;
  uint16_t* kp = dK + head + (size_t)kj * D;
  uint16_t* vp = dV + head + (size_t)kj * D;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      store_bf16x4(kp + 32 * cb + 8 * g + 4 * h, dka[cb][4 * g] * scale, dka[cb][4 * g + 1] * scale,
                   dka[cb][4 * g + 2] * scale, dka[cb][4 * g + 3] * scale);
      store_bf16x4(vp + 32 * cb + 8 * g + 4 * h, dva[cb][4 * g], dva[cb][4 * g + 1], dva[cb][4 * g + 2],
                   dva[cb][4 * g + 3]);
    }
  };
  body(item0);
  if constexpr (CAUSAL) {
    if (item1 >= 0) {
      __syncthreads();  // the next key tile's prologue rewrites the LDS
      body(item1);
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

template <int D, int BN, bool CAUSAL, bool TIES_ONLY>
static hipError_t launch_fwd_bn(const FwdArgs& a, hipStream_t st) {
  const int nqt = (a.N + 127) / 128;
  const int BH = a.B * a.H;
  hipLaunchKernelGGL((fwd_kernel<D, BN, CAUSAL, TIES_ONLY>), dim3(nqt * BH), dim3(256), 0, st,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.o32,
                     a.lse, a.ties, a.pbar_one, a.formed_ones, a.rowmax, BH, a.N, a.scale, a.stabilise,
                     a.beta, nqt);
  return hipGetLastError();
}

// The duplicate detector alone (no V tile, no P_bar V) streams 128-key tiles
// from N = 2048 on: half the barriers per key; measured on MI355X: sink
// (N = 2048) 31.8 -> 29.5 us, long_context (N = 8192, d = 128) 150.4 ->
// 131.9 us, while at N = 1024 the wider causal diagonal tile costs as much as
// it saves.  The (max, count) merge is exact and order-free, so the outputs
// are the same for either width.
template <int D, bool CAUSAL, bool TIES_ONLY>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t st) {
  if constexpr (TIES_ONLY) {
    if (a.N >= 2048) return launch_fwd_bn<D, 128, CAUSAL, true>(a, st);
    return launch_fwd_bn<D, 64, CAUSAL, true>(a, st);
  }
  return launch_fwd_bn<D, kFwdTile<D>, CAUSAL, false>(a, st);
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_fixed_t(const FwdArgs& a, hipStream_t st) {
  const int nqt = (a.N + 127) / 128;
  const int BH = a.B * a.H;
  constexpr int BN = kFwdTile<D>;
  // pass 1 (K alone) in tiles of twice the width (one stage) from N = 2048 on,
  // as the stand-alone detector
  if (a.N >= 2048)
    hipLaunchKernelGGL((fwd_fixed_kernel<D, BN, CAUSAL, 2 * BN>), dim3(nqt * BH), dim3(256), 0, st,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.o32,
                       a.lse, a.formed_ones, a.ties, a.pbar_one, BH, a.N, a.scale, a.beta, nqt);
  else
    hipLaunchKernelGGL((fwd_fixed_kernel<D, BN, CAUSAL, BN>), dim3(nqt * BH), dim3(256), 0, st,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.o32,
                       a.lse, a.formed_ones, a.ties, a.pbar_one, BH, a.N, a.scale, a.beta, nqt);
  return hipGetLastError();
}

template <bool TIES_ONLY>
static hipError_t launch_fwd_any(const FwdArgs& a, hipStream_t st) {
  if (a.D == 64) return a.causal ? launch_fwd_t<64, true, TIES_ONLY>(a, st) : launch_fwd_t<64, false, TIES_ONLY>(a, st);
  return a.causal ? launch_fwd_t<128, true, TIES_ONLY>(a, st) : launch_fwd_t<128, false, TIES_ONLY>(a, st);
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t st) {
  if (a.stabilise != 2) return launch_fwd_any<false>(a, st);
  // exact final shift: one kernel, the row's (max, count) first, then P_bar
  // formed once with the rule's shift
  if (a.D == 64) return a.causal ? launch_fwd_fixed_t<64, true>(a, st) : launch_fwd_fixed_t<64, false>(a, st);
  return a.causal ? launch_fwd_fixed_t<128, true>(a, st) : launch_fwd_fixed_t<128, false>(a, st);
}

hipError_t launch_tiecount(const FwdArgs& a, hipStream_t st) { return launch_fwd_any<true>(a, st); }

int fwd_key_tile(int D) { return D == 64 ? kFwdTile<64> : D == 128 ? kFwdTile<128> : 0; }

template <int D, bool CAUSAL>
static hipError_t launch_dq_t(const BwdArgs& a, hipStream_t st) {
  constexpr int BN = (D == 64 ? NSS_DQ_BN : 64);
  const int nqt = (a.N + 127) / 128;
  const int BH = a.B * a.H;
  if (a.o32)
    hipLaunchKernelGGL((bwd_dq_kernel<D, BN, CAUSAL, true>), dim3(nqt * BH), dim3(256), 0, st, (const uint16_t*)a.q,
                       (const uint16_t*)a.k, (const uint16_t*)a.v, (const void*)a.o32, (const uint16_t*)a.dO,
                       a.lse, (uint16_t*)a.dq, a.delta, BH, a.N, a.scale, nqt);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, BN, CAUSAL, false>), dim3(nqt * BH), dim3(256), 0, st,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.o, (const uint16_t*)a.dO,
                       a.lse, (uint16_t*)a.dq, a.delta, BH, a.N, a.scale, nqt);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_dkdv_t(const BwdArgs& a, hipStream_t st) {
  constexpr int BQ = (D == 64 ? NSS_DKDV_BQ : 32);
  const int nkt = (a.N + 127) / 128;
  const int BH = a.B * a.H;
  // causal: pack the key tiles of each XCD into one round of 2 workgroups per
  // CU (32 CUs per XCD) where they exceed it; nloc - single is made even so
  // that the paired tiles pair up exactly
  int grid = nkt * BH, single = -1;
  PairOrder ord{};
  if (CAUSAL && (BH & 7) == 0) {
    const int nloc = (BH >> 3) * nkt, per_round = 64;
    if (nloc > per_round) {
      int sg = nloc >= 2 * per_round ? 0 : 2 * per_round - nloc;
      if ((nloc - sg) & 1) ++sg;
      single = sg;
      grid = 8 * (sg + (nloc - sg) / 2);
      if (nloc <= 2 * per_round) place_pairs(ord, nloc, sg, BH >> 3, (a.N + BQ - 1) / BQ, 128 / BQ);
    }
  }
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, BQ, CAUSAL>), dim3(grid), dim3(256), 0, st, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dO, a.lse, a.delta,
                     (uint16_t*)a.dk, (uint16_t*)a.dv, BH, a.N, a.scale, nkt, single, ord);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t st) {
  if (a.D == 64) return a.causal ? launch_dq_t<64, true>(a, st) : launch_dq_t<64, false>(a, st);
  return a.causal ? launch_dq_t<128, true>(a, st) : launch_dq_t<128, false>(a, st);
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t st) {
  if (a.D == 64) return a.causal ? launch_dkdv_t<64, true>(a, st) : launch_dkdv_t<64, false>(a, st);
  return a.causal ? launch_dkdv_t<128, true>(a, st) : launch_dkdv_t<128, false>(a, st);
}

}  // namespace nss
