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
//   * the score tile is formed TRANSPOSED where a row statistic is needed
//     (keys on the MFMA row axis, the 32 queries on the lane axis), so the row
//     max, the duplicate count and the row sum are in-lane reductions plus one
//     exchange between the two 32-lane halves;
//   * the fp32 accumulator layout of one contraction is reused directly as the
//     bf16 B operand of the next (P_bar V, dS K, P^T dO, dS^T Q): the k index
//     of each MFMA is permuted to match, and the other operand is read from an
//     LDS copy stored transposed;
//   * K/V (forward, dQ pass) or Q/dO (dK/dV pass) tiles are staged through
//     LDS, double-buffered, one barrier per tile;
//   * causal work is ordered heaviest tile first.
//
// MFMA 32x32x16 lane layout (lane l, half h = l / 32):
//   A (32 x 16): lane l holds row l % 32, k = 8h .. 8h+7
//   B (16 x 32): lane l holds col l % 32, k = 8h .. 8h+7
//   C (32 x 32): element r of lane l is row 8(r/4) + 4h + r%4, col l % 32
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"

namespace nss {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// bf16 rounds x to exactly 1.0 (nearest even) iff 1 - 2^-9 <= x <= 1 + 2^-8;
// every P_bar here is at most 1 (plus exp2 rounding), so one compare decides.
constexpr float kBf16OneLow = 0.998046875f;

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor32f(float v) { return __shfl_xor(v, 32); }
__device__ __forceinline__ int xor32i(int v) { return __shfl_xor(v, 32); }

// eight fp32 accumulator values -> the bf16 B operand of the next contraction
__device__ __forceinline__ bf16x8 pack8(const f32x16& s, int base) {
  bf16x8 r;
#pragma unroll
  for (int t = 0; t < 8; t += 2) {
    bf16x2 p = __builtin_convertvector(f32x2{s[base + t], s[base + t + 1]}, bf16x2);
    r[t] = p[0];
    r[t + 1] = p[1];
  }
  return r;
}

// A operand from a transposed LDS tile T[c][n] (pitch P elements): row c, the
// 8 k slots of lane half h are n0 + 4h + {0..3} and n0 + 8 + 4h + {0..3}.
__device__ __forceinline__ bf16x8 lds_tr_operand(const uint16_t* row_c, int n0, int h) {
  u32x2 a = *reinterpret_cast<const u32x2*>(row_c + n0 + 4 * h);
  u32x2 b = *reinterpret_cast<const u32x2*>(row_c + n0 + 8 + 4 * h);
  return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}

// Stage rows [r0, r0+R) x D of a bf16 [N][D] matrix into LDS, row-major with
// pitch P; rows >= N become zeros.
template <int R, int D, int P>
__device__ __forceinline__ void load_rows(const uint16_t* __restrict__ src, int r0, int N, int tid,
                                          u32x4 (&reg)[(R * D / 8 + 255) / 256]) {
  constexpr int CH = D / 8, TOT = R * CH, PER = (TOT + 255) / 256;
#pragma unroll
  for (int c = 0; c < PER; ++c) {
    const int idx = tid + c * 256;
    const int row = idx / CH, ch = idx % CH;
    const int r = r0 + row;
    reg[c] = (idx < TOT && r < N) ? ld16(src + (size_t)r * D + ch * 8) : u32x4{0, 0, 0, 0};
  }
}
template <int R, int D, int P>
__device__ __forceinline__ void store_rows(uint16_t* dst, int tid, const u32x4 (&reg)[(R * D / 8 + 255) / 256]) {
  constexpr int CH = D / 8, TOT = R * CH, PER = (TOT + 255) / 256;
#pragma unroll
  for (int c = 0; c < PER; ++c) {
    const int idx = tid + c * 256;
    if (idx < TOT) {
      const int row = idx / CH, ch = idx % CH;
      *reinterpret_cast<u32x4*>(dst + row * P + ch * 8) = reg[c];
    }
  }
}

// Stage the same rows transposed: T[c][row] with pitch P (>= R, P % 4 == 0).
// A task is 4 consecutive rows x 8 columns: four 16-byte loads, eight 8-byte
// LDS stores.  Tasks are spread over the threads [t0, t0 + 256).
template <int R, int D>
struct TrTask {
  static constexpr int CH = D / 8, TOT = (R / 4) * CH, PER = (TOT + 255) / 256;
};
template <int R, int D>
__device__ __forceinline__ void load_rows_tr(const uint16_t* __restrict__ src, int r0, int N, int tid,
                                             u32x4 (&reg)[TrTask<R, D>::PER][4]) {
  constexpr int CH = TrTask<R, D>::CH, TOT = TrTask<R, D>::TOT, PER = TrTask<R, D>::PER;
#pragma unroll
  for (int c = 0; c < PER; ++c) {
    const int idx = tid + c * 256;
    const int rg = idx / CH, ch = idx % CH;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = r0 + 4 * rg + q;
      reg[c][q] = (idx < TOT && r < N) ? ld16(src + (size_t)r * D + ch * 8) : u32x4{0, 0, 0, 0};
    }
  }
}
template <int R, int D, int P>
__device__ __forceinline__ void store_rows_tr(uint16_t* dst, int tid, const u32x4 (&reg)[TrTask<R, D>::PER][4]) {
  constexpr int CH = TrTask<R, D>::CH, TOT = TrTask<R, D>::TOT, PER = TrTask<R, D>::PER;
#pragma unroll
  for (int c = 0; c < PER; ++c) {
    const int idx = tid + c * 256;
    if (idx < TOT) {
      const int rg = idx / CH, ch = idx % CH;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int p = e >> 1;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t lo = __builtin_amdgcn_perm(reg[c][1][p], reg[c][0][p], sel);
        const uint32_t hi = __builtin_amdgcn_perm(reg[c][3][p], reg[c][2][p], sel);
        *reinterpret_cast<u32x2*>(dst + (ch * 8 + e) * P + 4 * rg) = u32x2{lo, hi};
      }
    }
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

// ---------------------------------------------------------------------------
// Forward (and, with TIES_ONLY, the duplicate-max detector alone).
// One workgroup = 128 queries of one (b, h); 4 waves x 32 queries; KV tiles of
// 64 keys.  Per tile and wave: S^T = K Q^T (D/16 x 2 MFMAs), the online
// (max, count) merge and shift, P_bar = exp2(S t - m2), O^T += V^T P_bar^T.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool TIES_ONLY>
__global__ __launch_bounds__(256, 2) void fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int32_t* __restrict__ TIES,
    int32_t* __restrict__ PONE, int32_t* __restrict__ FORMED, float* __restrict__ ROWMAX, int BH, int N,
    float scale, int stabilise, float beta, int nqt) {
  constexpr int BM = 128, BN = 64, KP = D + 8, VP = BN + 4, NKK = D / 16, NCB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[TIES_ONLY ? 1 : 2][TIES_ONLY ? 8 : D * VP];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 31, h = lane >> 5;
  const int L = blockIdx.x;
  const int qt = CAUSAL ? (nqt - 1 - L / BH) : (L / BH);
  const int bh = L % BH;
  const size_t head = (size_t)bh * N * D;
  const int q0 = qt * BM, qw = q0 + 32 * w, qi = qw + li;
  const float t = scale * kLog2e;

  bf16x8 qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    qf[kk] = as_bf16x8(qi < N ? ld16(Q + head + (size_t)qi * D + 16 * kk + 8 * h) : u32x4{0, 0, 0, 0});

  const int kend = CAUSAL ? min(q0 + BM, N) : N;
  const int nkt = (kend + BN - 1) / BN;

  f32x16 oacc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) oacc[cb] = f32x16{};
  float m_run = -INFINITY, m2_run = -INFINITY, lsum = 0.f;
  int c_run = 0, ones = 0;
  const bool count_ones = FORMED != nullptr;

  u32x4 kreg[(BN * D / 8 + 255) / 256];
  u32x4 vreg[TrTask<BN, D>::PER][4];
  auto fetch = [&](int kt) {
    load_rows<BN, D, KP>(K + head, kt * BN, N, tid, kreg);
    if constexpr (!TIES_ONLY) load_rows_tr<BN, D>(V + head, kt * BN, N, tid, vreg);
  };
  auto commit = [&](int buf) {
    store_rows<BN, D, KP>(Ks[buf], tid, kreg);
    if constexpr (!TIES_ONLY) store_rows_tr<BN, D, VP>(Vt[buf], tid, vreg);
  };
  fetch(0);
  commit(0);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) fetch(kt + 1);
    const int k0 = kt * BN;
    const bool active = qw < N && (!CAUSAL || k0 <= qw + 31);
    if (active) {
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        const uint16_t* kp = &Ks[buf][(32 * kb + li) * KP + 8 * h];
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) s[kb] = mfma(as_bf16x8(ld16(kp + 16 * kk)), qf[kk], s[kb]);
      }
      const bool need_mask = (CAUSAL && k0 + BN - 1 > qw) || (k0 + BN > N);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
            if ((CAUSAL && key > qi) || key >= N) s[kb][r] = -INFINITY;
          }
      }
      // tile (max, count) on the raw fp32 dot products, then the running merge
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = fmaxf(mx, xor32f(mx));
      int cnt = 0;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) cnt += (s[kb][r] == mx) ? 1 : 0;
      cnt += xor32i(cnt);
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
        const float alpha = (m2_run == -INFINITY) ? 0.f : exp2f_fast(m2_run - m2);
        m2_run = m2;
        lsum *= alpha;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) oacc[cb] *= alpha;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = exp2f_fast(__builtin_fmaf(s[kb][r], t, -m2));
            s[kb][r] = p;
            lsum += p;
          }
        if (count_ones) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) ones += (s[kb][r] >= kBf16OneLow) ? 1 : 0;
        }
        bf16x8 pb[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          pb[kb][0] = pack8(s[kb], 0);
          pb[kb][1] = pack8(s[kb], 8);
        }
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const uint16_t* vp = &Vt[buf][(32 * cb + li) * VP];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int m = 0; m < 2; ++m)
              oacc[cb] = mfma(lds_tr_operand(vp, 32 * kb + 16 * m, h), pb[kb][m], oacc[cb]);
        }
      }
    }
    if (kt + 1 < nkt) commit(buf ^ 1);
    __syncthreads();
  }

  if (qw >= N) return;
  const size_t row = (size_t)bh * N + qi;
  if constexpr (TIES_ONLY) {
    if (h == 0 && qi < N) {
      TIES[row] = c_run;
      if (ROWMAX) ROWMAX[row] = scale * m_run;
    }
  } else {
    const float ltot = lsum + xor32f(lsum);
    const int ones_tot = ones + xor32i(ones);
    const float inv = 1.0f / ltot;
    if (qi < N) {
      uint16_t* op = O + head + (size_t)qi * D;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x2 a = __builtin_convertvector(f32x2{oacc[cb][4 * g] * inv, oacc[cb][4 * g + 1] * inv}, bf16x2);
          bf16x2 b = __builtin_convertvector(f32x2{oacc[cb][4 * g + 2] * inv, oacc[cb][4 * g + 3] * inv}, bf16x2);
          *reinterpret_cast<u32x2*>(op + 32 * cb + 8 * g + 4 * h) =
              u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
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
// Backward, query side: delta_i = sum_c dO_ic O_ic, then for each KV tile
// S^T = K Q^T, P = exp2(S t - lse2), dP^T = V dO^T, dS = P (dP - delta),
// dQ^T += K^T dS^T.  One workgroup = 128 queries; KV tiles of BN keys.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ Og, const uint16_t* __restrict__ dO, const float* __restrict__ LSE,
    uint16_t* __restrict__ dQ, float* __restrict__ DELTA, int BH, int N, float scale, int nqt) {
  constexpr int BM = 128, BN = (D == 64 ? 64 : 32), NKB = BN / 32, KP = D + 8, TP = BN + 4;
  constexpr int NKK = D / 16, NCB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][BN * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[2][D * TP];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 31, h = lane >> 5;
  const int L = blockIdx.x;
  const int qt = CAUSAL ? (nqt - 1 - L / BH) : (L / BH);
  const int bh = L % BH;
  const size_t head = (size_t)bh * N * D;
  const int q0 = qt * BM, qw = q0 + 32 * w, qi = qw + li;
  const float t = scale * kLog2e;

  bf16x8 qf[NKK], gf[NKK];
  float dl = 0.f;
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const size_t off = head + (size_t)qi * D + 16 * kk + 8 * h;
    const u32x4 z{0, 0, 0, 0};
    qf[kk] = as_bf16x8(qi < N ? ld16(Q + off) : z);
    gf[kk] = as_bf16x8(qi < N ? ld16(dO + off) : z);
    const bf16x8 of = as_bf16x8(qi < N ? ld16(Og + off) : z);
#pragma unroll
    for (int e = 0; e < 8; ++e) dl += (float)gf[kk][e] * (float)of[e];
  }
  dl += xor32f(dl);
  const float lse2 = qi < N ? LSE[(size_t)bh * N + qi] * kLog2e : 0.f;
  if (h == 0 && qi < N) DELTA[(size_t)bh * N + qi] = dl;

  const int kend = CAUSAL ? min(q0 + BM, N) : N;
  const int nkt = (kend + BN - 1) / BN;
  f32x16 dqa[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) dqa[cb] = f32x16{};

  u32x4 kreg[(BN * D / 8 + 255) / 256], vreg[(BN * D / 8 + 255) / 256];
  u32x4 treg[TrTask<BN, D>::PER][4];
  auto fetch = [&](int kt) {
    load_rows<BN, D, KP>(K + head, kt * BN, N, tid, kreg);
    load_rows<BN, D, KP>(V + head, kt * BN, N, tid, vreg);
    load_rows_tr<BN, D>(K + head, kt * BN, N, tid, treg);
  };
  auto commit = [&](int buf) {
    store_rows<BN, D, KP>(Ks[buf], tid, kreg);
    store_rows<BN, D, KP>(Vs[buf], tid, vreg);
    store_rows_tr<BN, D, TP>(Kt[buf], tid, treg);
  };
  fetch(0);
  commit(0);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) fetch(kt + 1);
    const int k0 = kt * BN;
    const bool active = qw < N && (!CAUSAL || k0 <= qw + 31);
    if (active) {
      f32x16 s[NKB], dp[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = f32x16{};
        dp[kb] = f32x16{};
        const uint16_t* kp = &Ks[buf][(32 * kb + li) * KP + 8 * h];
        const uint16_t* vp = &Vs[buf][(32 * kb + li) * KP + 8 * h];
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          s[kb] = mfma(as_bf16x8(ld16(kp + 16 * kk)), qf[kk], s[kb]);
          dp[kb] = mfma(as_bf16x8(ld16(vp + 16 * kk)), gf[kk], dp[kb]);
        }
      }
      const bool need_mask = (CAUSAL && k0 + BN - 1 > qw) || (k0 + BN > N);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[kb][r];
          if (need_mask) {
            const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
            if ((CAUSAL && key > qi) || key >= N) x = -INFINITY;
          }
          const float p = exp2f_fast(__builtin_fmaf(x, t, -lse2));
          s[kb][r] = p * (dp[kb][r] - dl);
        }
      bf16x8 db[NKB][2];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        db[kb][0] = pack8(s[kb], 0);
        db[kb][1] = pack8(s[kb], 8);
      }
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const uint16_t* tp = &Kt[buf][(32 * cb + li) * TP];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int m = 0; m < 2; ++m) dqa[cb] = mfma(lds_tr_operand(tp, 32 * kb + 16 * m, h), db[kb][m], dqa[cb]);
      }
    }
    if (kt + 1 < nkt) commit(buf ^ 1);
    __syncthreads();
  }

  if (qi >= N) return;
  uint16_t* qp = dQ + head + (size_t)qi * D;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x2 a = __builtin_convertvector(f32x2{dqa[cb][4 * g] * scale, dqa[cb][4 * g + 1] * scale}, bf16x2);
      bf16x2 b = __builtin_convertvector(f32x2{dqa[cb][4 * g + 2] * scale, dqa[cb][4 * g + 3] * scale}, bf16x2);
      *reinterpret_cast<u32x2*>(qp + 32 * cb + 8 * g + 4 * h) =
          u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
    }
}

// ---------------------------------------------------------------------------
// Backward, key side: one workgroup = 128 keys (4 waves x 32); query tiles of
// BQ rows.  Per tile: S = Q K^T (keys on the lane axis), P = exp2(S t - lse2),
// dP = dO V^T, dS = P (dP - delta), dV^T += dO^T P, dK^T += Q^T dS.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ DELTA,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int BH, int N, float scale) {
  constexpr int BK = 128, BQ = (D == 64 ? 64 : 32), NQB = BQ / 32, KP = D + 8, TP = BQ + 4;
  constexpr int NKK = D / 16, NCB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[2][BQ * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Gs[2][BQ * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Qt[2][D * TP];
  __shared__ __attribute__((aligned(16))) uint16_t Gt[2][D * TP];
  __shared__ __attribute__((aligned(16))) float Ls[2][BQ];
  __shared__ __attribute__((aligned(16))) float Ds[2][BQ];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 31, h = lane >> 5;
  const int L = blockIdx.x;
  const int kt = L / BH;   // causal: the first key tiles see the most queries
  const int bh = L % BH;
  const size_t head = (size_t)bh * N * D;
  const int k0 = kt * BK, kw = k0 + 32 * w, kj = kw + li;
  const float t = scale * kLog2e;

  bf16x8 kf[NKK], vf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const size_t off = head + (size_t)kj * D + 16 * kk + 8 * h;
    const u32x4 z{0, 0, 0, 0};
    kf[kk] = as_bf16x8(kj < N ? ld16(K + off) : z);
    vf[kk] = as_bf16x8(kj < N ? ld16(V + off) : z);
  }
  f32x16 dka[NCB], dva[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    dka[cb] = f32x16{};
    dva[cb] = f32x16{};
  }

  const int qstart = CAUSAL ? (k0 / BQ) : 0;
  const int nqt = (N + BQ - 1) / BQ;

  u32x4 qreg[(BQ * D / 8 + 255) / 256], greg[(BQ * D / 8 + 255) / 256];
  u32x4 qtr[TrTask<BQ, D>::PER][4], gtr[TrTask<BQ, D>::PER][4];
  float lreg = 0.f, dreg = 0.f;
  auto fetch = [&](int qt) {
    const int r0 = qt * BQ;
    load_rows<BQ, D, KP>(Q + head, r0, N, tid, qreg);
    load_rows<BQ, D, KP>(dO + head, r0, N, tid, greg);
    load_rows_tr<BQ, D>(Q + head, r0, N, tid, qtr);
    load_rows_tr<BQ, D>(dO + head, r0, N, tid, gtr);
    if (tid < BQ) {
      const int r = r0 + tid;
      lreg = r < N ? LSE[(size_t)bh * N + r] * kLog2e : INFINITY;   // rows past N: P = 0
      dreg = r < N ? DELTA[(size_t)bh * N + r] : 0.f;
    }
  };
  auto commit = [&](int buf) {
    store_rows<BQ, D, KP>(Qs[buf], tid, qreg);
    store_rows<BQ, D, KP>(Gs[buf], tid, greg);
    store_rows_tr<BQ, D, TP>(Qt[buf], tid, qtr);
    store_rows_tr<BQ, D, TP>(Gt[buf], tid, gtr);
    if (tid < BQ) {
      Ls[buf][tid] = lreg;
      Ds[buf][tid] = dreg;
    }
  };
  if (qstart < nqt && k0 < N) {
    fetch(qstart);
    commit(0);
  }
  __syncthreads();

  for (int qt = qstart; qt < nqt && k0 < N; ++qt) {
    const int buf = (qt - qstart) & 1;
    if (qt + 1 < nqt) fetch(qt + 1);
    const int r0 = qt * BQ;
    const bool active = kw < N && (!CAUSAL || r0 + BQ - 1 >= kw);
    if (active) {
      f32x16 s[NQB], dp[NQB];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        s[qb] = f32x16{};
        dp[qb] = f32x16{};
        const uint16_t* qp = &Qs[buf][(32 * qb + li) * KP + 8 * h];
        const uint16_t* gp = &Gs[buf][(32 * qb + li) * KP + 8 * h];
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          s[qb] = mfma(as_bf16x8(ld16(qp + 16 * kk)), kf[kk], s[qb]);
          dp[qb] = mfma(as_bf16x8(ld16(gp + 16 * kk)), vf[kk], dp[qb]);
        }
      }
      const bool need_mask = CAUSAL && r0 < kw + 31;
      bf16x8 pb[NQB][2], db[NQB][2];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int rl = 32 * qb + 8 * g + 4 * h;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&Ls[buf][rl]);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&Ds[buf][rl]);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int r = 4 * g + jj;
            float x = s[qb][r];
            if (need_mask && r0 + rl + jj < kj) x = -INFINITY;
            const float p = exp2f_fast(__builtin_fmaf(x, t, -l4[jj]));
            s[qb][r] = p;
            dp[qb][r] = p * (dp[qb][r] - d4[jj]);
          }
        }
        pb[qb][0] = pack8(s[qb], 0);
        pb[qb][1] = pack8(s[qb], 8);
        db[qb][0] = pack8(dp[qb], 0);
        db[qb][1] = pack8(dp[qb], 8);
      }
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const uint16_t* gt = &Gt[buf][(32 * cb + li) * TP];
        const uint16_t* qtp = &Qt[buf][(32 * cb + li) * TP];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            dva[cb] = mfma(lds_tr_operand(gt, 32 * qb + 16 * m, h), pb[qb][m], dva[cb]);
            dka[cb] = mfma(lds_tr_operand(qtp, 32 * qb + 16 * m, h), db[qb][m], dka[cb]);
          }
      }
    }
    if (qt + 1 < nqt) commit(buf ^ 1);
    __syncthreads();
  }

  if (kj >= N) return;
  uint16_t* kp = dK + head + (size_t)kj * D;
  uint16_t* vp = dV + head + (size_t)kj * D;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x2 a = __builtin_convertvector(f32x2{dka[cb][4 * g] * scale, dka[cb][4 * g + 1] * scale}, bf16x2);
      bf16x2 b = __builtin_convertvector(f32x2{dka[cb][4 * g + 2] * scale, dka[cb][4 * g + 3] * scale}, bf16x2);
      *reinterpret_cast<u32x2*>(kp + 32 * cb + 8 * g + 4 * h) =
          u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
      bf16x2 c = __builtin_convertvector(f32x2{dva[cb][4 * g], dva[cb][4 * g + 1]}, bf16x2);
      bf16x2 d = __builtin_convertvector(f32x2{dva[cb][4 * g + 2], dva[cb][4 * g + 3]}, bf16x2);
      *reinterpret_cast<u32x2*>(vp + 32 * cb + 8 * g + 4 * h) =
          u32x2{__builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool TIES_ONLY>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t st) {
  const int nqt = (a.N + 127) / 128;
  const int BH = a.B * a.H;
  hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, TIES_ONLY>), dim3(nqt * BH), dim3(256), 0, st,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.lse,
                     a.ties, a.pbar_one, a.formed_ones, a.rowmax, BH, a.N, a.scale, a.stabilise, a.beta, nqt);
  return hipGetLastError();
}

template <bool TIES_ONLY>
static hipError_t launch_fwd_any(const FwdArgs& a, hipStream_t st) {
  if (a.D == 64) return a.causal ? launch_fwd_t<64, true, TIES_ONLY>(a, st) : launch_fwd_t<64, false, TIES_ONLY>(a, st);
  return a.causal ? launch_fwd_t<128, true, TIES_ONLY>(a, st) : launch_fwd_t<128, false, TIES_ONLY>(a, st);
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t st) { return launch_fwd_any<false>(a, st); }
hipError_t launch_tiecount(const FwdArgs& a, hipStream_t st) { return launch_fwd_any<true>(a, st); }

template <int D, bool CAUSAL>
static hipError_t launch_dq_t(const BwdArgs& a, hipStream_t st) {
  const int nqt = (a.N + 127) / 128;
  const int BH = a.B * a.H;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(nqt * BH), dim3(256), 0, st, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.o, (const uint16_t*)a.dO,
                     a.lse, (uint16_t*)a.dq, a.delta, BH, a.N, a.scale, nqt);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_dkdv_t(const BwdArgs& a, hipStream_t st) {
  const int nkt = (a.N + 127) / 128;
  const int BH = a.B * a.H;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(nkt * BH), dim3(256), 0, st, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dO, a.lse, a.delta,
                     (uint16_t*)a.dk, (uint16_t*)a.dv, BH, a.N, a.scale);
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
