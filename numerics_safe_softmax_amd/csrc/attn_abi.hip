// attn_abi.hip -- the extern "C" entry points declared in include/attn.h:
// argument validation (before any HIP call), the gfx950 device check, and the
// kernel launches on the caller's stream.  The library allocates nothing and
// never synchronises.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "attn.h"
#include "attn_launch.h"

namespace {

struct Span {
  const void* p;
  size_t bytes;
};

bool overlaps(const Span& a, const Span& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

bool misaligned(const void* p) { return p && ((uintptr_t)p & 15u) != 0; }

// Shape, head size, scale and beta; sets *empty when there is nothing to do.
int check_scalars(int B, int H, int N, int D, float scale, int check_beta, float beta, bool* empty) {
  if (B < 0 || H < 0 || N < 0) return ATTN_E_SHAPE;
  const long long bh = (long long)B * H;
  if (bh > 0 && N > 0) {
    // row and key indices are 32-bit (kept well clear of overflow: N < 2^24;
    // element offsets are 64-bit), and a launch holds fewer than 2^32
    // work-items, i.e. fewer than 2^24 workgroups of 256 for the
    // B * H * ceil(N / 128) row tiles of every pass
    if (N >= (1 << 24)) return ATTN_E_SHAPE;
    if (bh >= (1LL << 24) || bh * ((N + 127) / 128) >= (1LL << 24)) return ATTN_E_SHAPE;
  }
  if (D != 64 && D != 128) return ATTN_E_HEADDIM;
  if (!std::isfinite(scale) || !(scale > 0.f)) return ATTN_E_SCALE;
  if (check_beta && (!std::isfinite(beta) || !(beta > 1.f))) return ATTN_E_BETA;
  *empty = bh == 0 || N == 0;
  return ATTN_OK;
}

// outputs may not overlap inputs or each other
int check_alias(const Span* in, int nin, const Span* out, int nout) {
  for (int o = 0; o < nout; ++o) {
    for (int i = 0; i < nin; ++i)
      if (overlaps(out[o], in[i])) return ATTN_E_ALIAS;
    for (int p = o + 1; p < nout; ++p)
      if (overlaps(out[o], out[p])) return ATTN_E_ALIAS;
  }
  return ATTN_OK;
}

int check_align(const void* const* ptrs, int n) {
  for (int i = 0; i < n; ++i)
    if (misaligned(ptrs[i])) return ATTN_E_ALIGN;
  return ATTN_OK;
}

// per-device cache: 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_arch[64];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_E_DEVICE;
  if (dev < 0 || dev >= 64) return ATTN_E_DEVICE;
  int known = g_arch[dev].load(std::memory_order_relaxed);
  if (known == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_E_DEVICE;
    known = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch[dev].store(known, std::memory_order_relaxed);
  }
  return known == 1 ? ATTN_OK : ATTN_E_DEVICE;
}

int launched(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_E_DEVICE; }

}  // namespace

extern "C" {

int attn_abi_version(void) { return 5; }

int attn_fwd_key_tile(int D) {
  const int w = nss::fwd_key_tile(D);
  return w > 0 ? w : ATTN_E_HEADDIM;
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_E_NULLPTR: return "a required pointer is NULL";
    case ATTN_E_SHAPE: return "B, H or N negative, N of 2^24 or more, or B*H*ceil(N/128) of 2^24 or more";
    case ATTN_E_HEADDIM: return "head size D must be 64 or 128";
    case ATTN_E_BETA: return "with stabilise set, beta must be finite and greater than 1";
    case ATTN_E_SCALE: return "scale must be finite and greater than 0";
    case ATTN_E_ALIGN: return "every pointer must be 16-byte aligned";
    case ATTN_E_ALIAS: return "an output overlaps an input or another output";
    case ATTN_E_WORKSPACE: return "workspace is NULL, misaligned or smaller than attn_bwd_workspace_bytes";
    case ATTN_E_DEVICE: return "not a gfx950 device, or a HIP launch failed";
    case ATTN_E_MODE: return "stabilise must be 0 (plain), 1 (online shift) or 2 (exact final shift)";
    default: return "unknown attn_status";
  }
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int32_t* ties,
             int32_t* pbar_one, int32_t* formed_ones, int B, int H, int N, int D, float scale, int causal,
             int stabilise, float beta, void* stream) {
  bool empty = false;
  int st = check_scalars(B, H, N, D, scale, stabilise != 0, beta, &empty);
  if (st == ATTN_OK && (stabilise < 0 || stabilise > 2)) st = ATTN_E_MODE;
  if (st != ATTN_OK || empty) return st;
  if (!q || !k || !v || !o || !lse) return ATTN_E_NULLPTR;
  const void* ptrs[] = {q, k, v, o, lse, ties, pbar_one, formed_ones};
  if ((st = check_align(ptrs, 8)) != ATTN_OK) return st;
  const size_t tb = (size_t)B * H * N * D * 2, rb = (size_t)B * H * N * 4;
  const Span in[] = {{q, tb}, {k, tb}, {v, tb}};
  const Span out[] = {{o, tb}, {lse, rb}, {ties, rb}, {pbar_one, rb}, {formed_ones, rb}};
  if ((st = check_alias(in, 3, out, 5)) != ATTN_OK) return st;
  if ((st = check_device()) != ATTN_OK) return st;
  nss::FwdArgs a{q, k, v, o, nullptr, lse, ties, pbar_one, formed_ones, nullptr, B, H, N, D, scale,
                 causal ? 1 : 0, stabilise, beta};
  return launched(nss::launch_fwd(a, (hipStream_t)stream));
}

int attn_fwd_o32(const void* q, const void* k, const void* v, void* o, float* o32, float* lse, int32_t* ties,
                 int32_t* pbar_one, int32_t* formed_ones, int B, int H, int N, int D, float scale, int causal,
                 int stabilise, float beta, void* stream) {
  bool empty = false;
  int st = check_scalars(B, H, N, D, scale, stabilise != 0, beta, &empty);
  if (st == ATTN_OK && (stabilise < 0 || stabilise > 2)) st = ATTN_E_MODE;
  if (st != ATTN_OK || empty) return st;
  if (!q || !k || !v || !o || !o32 || !lse) return ATTN_E_NULLPTR;
  const void* ptrs[] = {q, k, v, o, o32, lse, ties, pbar_one, formed_ones};
  if ((st = check_align(ptrs, 9)) != ATTN_OK) return st;
  const size_t tb = (size_t)B * H * N * D * 2, rb = (size_t)B * H * N * 4;
  const Span in[] = {{q, tb}, {k, tb}, {v, tb}};
  const Span out[] = {{o, tb}, {o32, 2 * tb}, {lse, rb}, {ties, rb}, {pbar_one, rb}, {formed_ones, rb}};
  if ((st = check_alias(in, 3, out, 6)) != ATTN_OK) return st;
  if ((st = check_device()) != ATTN_OK) return st;
  nss::FwdArgs a{q, k, v, o, o32, lse, ties, pbar_one, formed_ones, nullptr, B, H, N, D, scale,
                 causal ? 1 : 0, stabilise, beta};
  return launched(nss::launch_fwd(a, (hipStream_t)stream));
}

int attn_tiecount(const void* q, const void* k, int32_t* ties, float* rowmax, int B, int H, int N, int D,
                  float scale, int causal, void* stream) {
  bool empty = false;
  int st = check_scalars(B, H, N, D, scale, 0, 0.f, &empty);
  if (st != ATTN_OK || empty) return st;
  if (!q || !k || !ties) return ATTN_E_NULLPTR;
  const void* ptrs[] = {q, k, ties, rowmax};
  if ((st = check_align(ptrs, 4)) != ATTN_OK) return st;
  const size_t tb = (size_t)B * H * N * D * 2, rb = (size_t)B * H * N * 4;
  const Span in[] = {{q, tb}, {k, tb}};
  const Span out[] = {{ties, rb}, {rowmax, rb}};
  if ((st = check_alias(in, 2, out, 2)) != ATTN_OK) return st;
  if ((st = check_device()) != ATTN_OK) return st;
  nss::FwdArgs a{q, k, nullptr, nullptr, nullptr, nullptr, ties, nullptr, nullptr, rowmax, B, H, N, D,
                 scale, causal ? 1 : 0, 0, 2.f};
  return launched(nss::launch_tiecount(a, (hipStream_t)stream));
}

int attn_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                void* dq, float* delta, int B, int H, int N, int D, float scale, int causal, void* stream) {
  bool empty = false;
  int st = check_scalars(B, H, N, D, scale, 0, 0.f, &empty);
  if (st != ATTN_OK || empty) return st;
  if (!q || !k || !v || !o || !dO || !lse || !dq || !delta) return ATTN_E_NULLPTR;
  const void* ptrs[] = {q, k, v, o, dO, lse, dq, delta};
  if ((st = check_align(ptrs, 8)) != ATTN_OK) return st;
  const size_t tb = (size_t)B * H * N * D * 2, rb = (size_t)B * H * N * 4;
  const Span in[] = {{q, tb}, {k, tb}, {v, tb}, {o, tb}, {dO, tb}, {lse, rb}};
  const Span out[] = {{dq, tb}, {delta, rb}};
  if ((st = check_alias(in, 6, out, 2)) != ATTN_OK) return st;
  if ((st = check_device()) != ATTN_OK) return st;
  nss::BwdArgs a{q, k, v, o, dO, nullptr, lse, dq, nullptr, nullptr, delta, B, H, N, D, scale, causal ? 1 : 0};
  return launched(nss::launch_bwd_dq(a, (hipStream_t)stream));
}

int attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                  const float* delta, void* dk, void* dv, int B, int H, int N, int D, float scale, int causal,
                  void* stream) {
  bool empty = false;
  int st = check_scalars(B, H, N, D, scale, 0, 0.f, &empty);
  if (st != ATTN_OK || empty) return st;
  if (!q || !k || !v || !dO || !lse || !delta || !dk || !dv) return ATTN_E_NULLPTR;
  const void* ptrs[] = {q, k, v, dO, lse, delta, dk, dv};
  if ((st = check_align(ptrs, 8)) != ATTN_OK) return st;
  const size_t tb = (size_t)B * H * N * D * 2, rb = (size_t)B * H * N * 4;
  const Span in[] = {{q, tb}, {k, tb}, {v, tb}, {dO, tb}, {lse, rb}, {delta, rb}};
  const Span out[] = {{dk, tb}, {dv, tb}};
  if ((st = check_alias(in, 6, out, 2)) != ATTN_OK) return st;
  if ((st = check_device()) != ATTN_OK) return st;
  nss::BwdArgs a{q, k, v, nullptr, dO, nullptr, lse, nullptr, dk, dv, const_cast<float*>(delta), B, H, N, D, scale,
                 causal ? 1 : 0};
  return launched(nss::launch_bwd_dkdv(a, (hipStream_t)stream));
}

size_t attn_bwd_workspace_bytes(int B, int H, int N, int D) {
  (void)B; (void)H; (void)N; (void)D;
  return 0;  // the two-pass backward keeps everything in registers and LDS
}

namespace {

// validation shared by attn_bwd and attn_bwd_o32 (o: bf16 O, or fp32 O when o32)
int bwd_entry(const void* q, const void* k, const void* v, const void* o, bool o32, const void* dO,
              const float* lse, void* dq, void* dk, void* dv, float* delta, void* workspace, size_t workspace_bytes,
              int B, int H, int N, int D, float scale, int causal, int stabilise, float beta, void* stream) {
  bool empty = false;
  int st = check_scalars(B, H, N, D, scale, stabilise != 0, beta, &empty);
  if (st == ATTN_OK && (stabilise < 0 || stabilise > 2)) st = ATTN_E_MODE;
  if (st != ATTN_OK || empty) return st;
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv || !delta) return ATTN_E_NULLPTR;
  const size_t need = attn_bwd_workspace_bytes(B, H, N, D);
  if (need && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 15u) != 0)) return ATTN_E_WORKSPACE;
  const void* ptrs[] = {q, k, v, o, dO, lse, dq, dk, dv, delta};
  if ((st = check_align(ptrs, 10)) != ATTN_OK) return st;
  const size_t tb = (size_t)B * H * N * D * 2, rb = (size_t)B * H * N * 4;
  const Span in[] = {{q, tb}, {k, tb}, {v, tb}, {o, o32 ? 2 * tb : tb}, {dO, tb}, {lse, rb}};
  const Span out[] = {{dq, tb}, {dk, tb}, {dv, tb}, {delta, rb}};
  if ((st = check_alias(in, 6, out, 4)) != ATTN_OK) return st;
  if ((st = check_device()) != ATTN_OK) return st;
  nss::BwdArgs a{q, k, v, o32 ? nullptr : o, dO, o32 ? static_cast<const float*>(o) : nullptr, lse, dq, dk, dv,
                 delta, B, H, N, D, scale, causal ? 1 : 0};
  if ((st = launched(nss::launch_bwd_dq(a, (hipStream_t)stream))) != ATTN_OK) return st;
  return launched(nss::launch_bwd_dkdv(a, (hipStream_t)stream));
}

}  // namespace

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
             void* dq, void* dk, void* dv, float* delta, void* workspace, size_t workspace_bytes, int B, int H, int N,
             int D, float scale, int causal, int stabilise, float beta, void* stream) {
  return bwd_entry(q, k, v, o, false, dO, lse, dq, dk, dv, delta, workspace, workspace_bytes, B, H, N, D, scale,
                   causal, stabilise, beta, stream);
}

int attn_bwd_o32(const void* q, const void* k, const void* v, const float* o32, const void* dO, const float* lse,
                 void* dq, void* dk, void* dv, float* delta, void* workspace, size_t workspace_bytes, int B, int H,
                 int N, int D, float scale, int causal, int stabilise, float beta, void* stream) {
  return bwd_entry(q, k, v, o32, true, dO, lse, dq, dk, dv, delta, workspace, workspace_bytes, B, H, N, D, scale,
                   causal, stabilise, beta, stream);
}

}  // extern "C"
