/*
 * attn.h -- C ABI of a BF16 fused softmax-attention library for AMD MI355X
 * (gfx950), with the duplicate-max ("stabilised") safe softmax as a
 * switchable mode.
 *
 * The method (web pages on Qiu & Yao, "Why Low-Precision Transformer Training
 * Fails: An Analysis on Flash Attention", arXiv 2510.04212):
 *   - itsolotime.com/archives/23922, section "机制解释二" (origin of the bias):
 *     the forward forms P_bar = exp(S - m), P = P_bar / rowsum(P_bar),
 *     O = P V; when a row of S reaches its maximum more than once, P_bar holds
 *     several entries exactly equal to 1, the trigger of the bias.
 *   - same page, section "极简修复方案" (minimal fix): count how often the row
 *     maximum rm occurs (rs); when rs > 1 the shift becomes beta * rm for
 *     rm > 0 (beta > 1) or 0 for rm < 0, otherwise it stays rm, so the largest
 *     P_bar entry of a repeated-max row falls below 1; softmax is unchanged by
 *     a per-row shift in exact arithmetic.
 *   - 91haoming.cn/news/show-608006, section 三: the backward's delta is the
 *     row-sum of an element-wise product, delta_i = sum_c dO_ic O_ic, and the
 *     backward forms dP.
 *
 * Conventions shared by every entry point
 *   Layout   q, k, v, o, dO, dq, dk, dv are bf16 (IEEE bfloat16 bits: 1 sign,
 *            8 exponent, 7 fraction bits), contiguous row-major [B][H][N][D];
 *            self-attention, the same N for queries and keys.  Per-row vectors
 *            (lse, delta, ties, ...) are contiguous [B][H][N].  All pointers
 *            are device pointers, 16-byte aligned.
 *   Causal   query i sees keys j <= i (top-left aligned); otherwise all N keys.
 *   Scores   S_ij = scale * (q_i . k_j); scale must be finite and > 0.  The
 *            duplicate test compares the raw fp32 dot products q_i . k_j as
 *            the kernel forms them (bf16 MFMA, fp32 accumulation); with
 *            scale > 0 this is the same order as S.
 *   Shapes   B, H, N >= 0 (B*H*N == 0 is a no-op returning ATTN_OK); any
 *            N >= 1 (ragged tiles are masked); D in {64, 128}; N below 2^24
 *            and B*H*ceil(N/128) below 2^24 (one launch of 256-thread
 *            workgroups holds fewer than 2^32 work-items).  Element offsets
 *            are 64-bit, so a tensor may exceed 2^31 elements (4 GiB) and
 *            the shape limits admit more than the 288 GB of one device.
 *   Ownership  The caller allocates and owns every buffer.  The library never
 *            allocates, frees or synchronises; it keeps no state between calls
 *            except a per-device cache of the device's architecture.  Inputs
 *            are read only; outputs are fully overwritten; no output may
 *            overlap an input or another output.
 *   Errors   Arguments are validated before any HIP call; on error nothing is
 *            launched and a negative attn_status is returned.  A device that
 *            is not gfx950, or a failed launch, returns ATTN_E_DEVICE.  Work
 *            is asynchronous on `stream` (a hipStream_t; NULL = the default
 *            stream), so faults surface at the caller's next synchronisation.
 *            No C++ exception crosses this interface.
 */
#ifndef NSS_ATTN_H
#define NSS_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_E_NULLPTR = -1,   /* a required pointer is NULL                          */
  ATTN_E_SHAPE = -2,     /* B, H or N negative, N >= 2^24 or B*H*ceil(N/128) >= 2^24 */
  ATTN_E_HEADDIM = -3,   /* D not in {64, 128}                                  */
  ATTN_E_BETA = -4,      /* stabilise != 0 and beta not finite or not > 1       */
  ATTN_E_SCALE = -5,     /* scale not finite or not > 0                         */
  ATTN_E_ALIGN = -6,     /* a pointer is not 16-byte aligned                    */
  ATTN_E_ALIAS = -7,     /* an output overlaps an input or another output       */
  ATTN_E_WORKSPACE = -8, /* workspace smaller than attn_bwd_workspace_bytes, or misaligned */
  ATTN_E_DEVICE = -9,    /* not a gfx950 device, or a HIP launch failed         */
  ATTN_E_MODE = -10      /* stabilise not 0, 1 or 2                             */
} attn_status;

/* Values of the `stabilise` argument. */
enum {
  ATTN_PLAIN = 0,        /* plain safe softmax: shift = running row max              */
  ATTN_STAB_ONLINE = 1,  /* duplicate-max shift from the running (max, count)        */
  ATTN_STAB_EXACT = 2    /* duplicate-max shift from the whole row's final (max,     */
                         /* count): two passes over the keys, no transient P_bar == 1 */
};

/*
 * attn_fwd -- fused attention forward with the online (max, count) merge.
 *
 * Computes, per row i and over its visible keys, S = scale * q_i . k_j, the
 * row maximum rm and how many keys reach it rs (merged across KV tiles as a
 * (max, count) pair: the larger max keeps its count, equal maxima add), the
 * shift m (stabilise == 0: m = rm; stabilise != 0: the rule of
 * itsolotime.com/archives/23922, section "极简修复方案"), P_bar = exp(S - m),
 * O = (P_bar V) / rowsum(P_bar) and LSE = m + ln rowsum(P_bar)
 * (section "机制解释二" of the same page).  The shift is applied online: while a
 * tile is processed, m comes from the running (max, count).  P_bar is formed
 * in fp32 and rounded to bf16 (nearest even) as the operand of P_bar V; O is
 * normalised by the sum of those bf16 operands (P = P_bar / rowsum(P_bar) with
 * the P_bar that P_bar V consumes, so O's weights sum to 1), while LSE takes
 * the sum of the fp32 values.
 *
 *   q, k, v      in   bf16 [B][H][N][D]
 *   o            out  bf16 [B][H][N][D]
 *   lse          out  fp32 [B][H][N], natural-log log-sum-exp of S (the
 *                     backward's input)
 *   ties         out  int32 [B][H][N] or NULL: rs, the final duplicate count
 *   pbar_one     out  int32 [B][H][N] or NULL: 1 when the largest entry of the
 *                     final-shift P_bar, exp(rm - m), rounds (bf16, nearest
 *                     even) to exactly 1.0, else 0
 *   formed_ones  out  int32 [B][H][N] or NULL: how many bf16 P_bar operands
 *                     equal to 1.0 the kernel actually fed to P_bar V (a tie
 *                     split across KV tiles forms one before its duplicate is
 *                     seen)
 *   stabilise    ATTN_PLAIN (0): plain safe softmax, online.
 *                ATTN_STAB_ONLINE (1): the duplicate-max shift, online: while a
 *                tile is processed the shift follows the running (max, count),
 *                so a duplicate that arrives in a later KV tile than the first
 *                occurrence leaves one transient exact 1 in P_bar (rescaled
 *                away afterwards; counted in formed_ones).
 *                ATTN_STAB_EXACT (2): the duplicate-max shift from each row's
 *                final (max, count): one launch, in which each workgroup
 *                first merges every KV tile of its rows (writing ties and
 *                pbar_one; the shift stays on chip), then forms every P_bar
 *                entry once with that shift,
 *                so no entry of a repeated-max row ever equals 1 (the rule of
 *                the minimal-fix section applied to the whole row, as written),
 *                and formed_ones counts exactly the entries whose bf16 rounding
 *                is 1 under the final shift.
 *                Other values: ATTN_E_MODE.
 *   beta         the rule's factor (> 1, finite) when stabilise != 0; ignored
 *                otherwise
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int32_t* ties, int32_t* pbar_one, int32_t* formed_ones,
             int B, int H, int N, int D, float scale, int causal, int stabilise,
             float beta, void* stream);

/*
 * attn_fwd_o32 -- attn_fwd that also returns O before its bf16 rounding.
 *
 * itsolotime.com/archives/23922, section "核心发现": training is stable again
 * once the P behind dP comes from a path of higher precision (or a
 * numerically equivalent, different one).  In this backward the forward's
 * rounding reaches dS = P o (dP - delta) through delta = rowsum(dO o O)
 * (91haoming.cn/news/show-608006, section 三); the fp32 O written here lets
 * attn_bwd_o32 form delta without O's bf16 rounding.  Everything else, the
 * arguments included, is as attn_fwd.
 *
 *   o32   out  fp32 [B][H][N][D]: O = O_acc / l before rounding to bf16
 *              (o holds the same values rounded to nearest even)
 */
int attn_fwd_o32(const void* q, const void* k, const void* v, void* o, float* o32, float* lse,
                 int32_t* ties, int32_t* pbar_one, int32_t* formed_ones,
                 int B, int H, int N, int D, float scale, int causal, int stabilise,
                 float beta, void* stream);

/*
 * attn_bwd_workspace_bytes -- size of the workspace attn_bwd needs: 0 for
 * every shape.  The backward keeps every intermediate in registers and LDS
 * (two passes: attn_bwd_dq then attn_bwd_dkdv; a one-pass form with dQ added
 * into an fp32 workspace by atomics measured slower on MI355X).  The query and
 * the workspace arguments are part of the interface so that a caller that
 * sizes the workspace by this call is correct whatever it returns.
 */
size_t attn_bwd_workspace_bytes(int B, int H, int N, int D);

/*
 * attn_bwd -- gradient of sum(dO * O) with respect to q, k and v.
 *
 * Runs attn_bwd_dq then attn_bwd_dkdv on `stream`.  With P = exp(S - lse):
 * delta_i = sum_c dO_ic O_ic (91haoming.cn/news/show-608006, section 三: a
 * row-sum of an element-wise product), dP = dO V^T, dS = P o (dP - delta),
 * dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO.  P is recomputed from the
 * forward's lse, which carries the forward's shift, so the arithmetic is the
 * same in every mode; `stabilise` and `beta` are validated as for attn_fwd
 * and otherwise unused.  Every output is reproducible bit for bit.
 *
 *   q, k, v, o, dO  in   bf16 [B][H][N][D] (o from attn_fwd)
 *   lse             in   fp32 [B][H][N] from attn_fwd
 *   dq, dk, dv      out  bf16 [B][H][N][D]
 *   delta           out  fp32 [B][H][N]: rowsum(dO o O), kept for the caller
 *   workspace       at least attn_bwd_workspace_bytes(B, H, N, D) bytes of
 *                   caller-owned device scratch, 16-byte aligned, contents
 *                   undefined on entry and on exit (NULL with 0 bytes where
 *                   that size is 0, as it is for every shape here); a
 *                   smaller or misaligned one is ATTN_E_WORKSPACE
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
             const float* lse, void* dq, void* dk, void* dv, float* delta,
             void* workspace, size_t workspace_bytes,
             int B, int H, int N, int D, float scale, int causal, int stabilise,
             float beta, void* stream);

/*
 * attn_bwd_o32 -- attn_bwd with delta_i = sum_c dO_ic O_ic taken from the fp32
 * O of attn_fwd_o32 (the high-precision delta path; see attn_fwd_o32).  dQ,
 * dK and dV follow from that delta exactly as in attn_bwd.
 *
 *   o32   in   fp32 [B][H][N][D] from attn_fwd_o32; other arguments as attn_bwd
 */
int attn_bwd_o32(const void* q, const void* k, const void* v, const float* o32, const void* dO,
                 const float* lse, void* dq, void* dk, void* dv, float* delta,
                 void* workspace, size_t workspace_bytes,
                 int B, int H, int N, int D, float scale, int causal, int stabilise,
                 float beta, void* stream);

/*
 * attn_bwd_dq -- first pass of attn_bwd: delta and dQ, one pass per query
 * tile over its visible keys (recomputing S and dP).  Arguments as attn_bwd.
 */
int attn_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dO,
                const float* lse, void* dq, float* delta,
                int B, int H, int N, int D, float scale, int causal, void* stream);

/*
 * attn_bwd_dkdv -- second pass of attn_bwd: dK and dV, one pass per key tile
 * over the queries that see it.  `delta` is read (attn_bwd_dq's output).
 */
int attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                  const float* lse, const float* delta, void* dk, void* dv,
                  int B, int H, int N, int D, float scale, int causal, void* stream);

/*
 * attn_tiecount -- the duplicate-max detector alone
 * (itsolotime.com/archives/23922, section "极简修复方案": whether, and how
 * often, the maximum of a row of S repeats).
 *
 *   q, k     in   bf16 [B][H][N][D]
 *   ties     out  int32 [B][H][N]: rs over the visible keys
 *   rowmax   out  fp32 [B][H][N] or NULL: rm = scale * max_j (q_i . k_j),
 *                 the fp32 product of scale and the raw fp32 maximum
 */
int attn_tiecount(const void* q, const void* k, int32_t* ties, float* rowmax,
                  int B, int H, int N, int D, float scale, int causal, void* stream);

/*
 * attn_fwd_key_tile -- keys per KV tile of attn_fwd and attn_fwd_o32 for head
 * size D: 64 at D = 64, 32 at D = 128; ATTN_E_HEADDIM for any other D.  No
 * device call.  The online modes (ATTN_PLAIN, ATTN_STAB_ONLINE) merge the
 * running (max, count) and move the shift once per tile (the rule of
 * itsolotime.com/archives/23922, section "极简修复方案", applied to the running
 * pair of the tiled computation that 91haoming.cn/news/show-608006 describes
 * in section 三), so which P_bar entries are transiently formed as 1
 * (formed_ones) depends on this width; ATTN_STAB_EXACT and every other output
 * (up to rounding) do not.
 */
int attn_fwd_key_tile(int D);

/* Static, human-readable text for an attn_status value. */
const char* attn_status_string(int status);

/* ABI version of this header (incremented on any signature change). */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NSS_ATTN_H */
