/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library libfa.so.
 *
 * The library computes exact scaled-dot-product attention the FlashAttention
 * way: the query rows are cut into tiles, key/value tiles are streamed through
 * on-chip memory, and every score tile is folded at once into per-row
 * online-softmax state, so that no N_q x N_kv score or probability matrix is
 * ever written to device memory.
 *
 * Pages cited (title, section):
 *   [BLOG] "AI infra. 一层全看懂(五)Flash Attention:AI编译优化的集大成者"
 *   [KB]   "FlashAttention：为什么少搬数据，反而算得更快"
 *   [NEWS] "FlashAttention技术原理详解：通过内存优化加速注意力计算"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout ([KB] §08, the q/k/v layout [batch, heads, sequence, head_dim]):
 *   q, o, dO, dq : [B, Hq,  N_q,  d]   contiguous, row-major, d fastest
 *   k, v, dk, dv : [B, Hkv, N_kv, d]   contiguous, row-major, d fastest
 *   lse          : [B, Hq,  N_q]       float32, always
 * Heads ([NEWS]: MHA / MQA / GQA): Hq must be a multiple of Hkv; query head h
 *   reads key/value head h / (Hq / Hkv). Hkv == Hq is MHA, Hkv == 1 is MQA.
 * Scale: S = scale * Q K^T; scale must be finite and > 0 (1/sqrt(d) is usual).
 * Causal ([KB] §02: the mask is part of the real computation): query row i
 *   sees key j iff j <= i + (N_kv - N_q) (aligned to the bottom-right corner;
 *   for N_q == N_kv that is j <= i, for N_q == 1 every key is visible).
 *   A row that sees no key gets O = 0, LSE = -inf and passes no gradient.
 * LSE ([KB] §05, the row statistic the backward rebuilds P from): natural-log
 *   log-sum-exp of the scaled, masked score row, m + ln(l) in the notation
 *   of [KB] §04.
 * dtypes: FA_F32 (forward only), FA_F16, FA_BF16. Outputs have the input
 *   dtype; all accumulation is float32; float32 -> 16-bit conversions round
 *   to nearest even.
 * Head dim d: 64 or 128. Sizes: N_kv * d < 2^29 (one head's K or V under
 *   2 GiB) and B * H * N < 2^31; larger problems return FA_ERR_UNSUPPORTED.
 *   The query side (q, o, dO, dq, lse) is addressed with 64-bit offsets, so
 *   one head's Q may exceed 4 GiB.
 * Pointers: device pointers, 16-byte aligned; the workspace 256-byte aligned.
 *   Outputs must not overlap inputs. Every output element is overwritten.
 * Ownership: the caller allocates and frees every buffer, including the
 *   workspace (size from fa_*_workspace_size). The library allocates nothing,
 *   frees nothing and keeps no pointer after a call returns.
 * Execution: every call only enqueues work on `stream` (NULL = the default
 *   stream) and returns; order consumers by stream. Calls are re-entrant; the
 *   library has no global mutable state.
 * Errors: arguments are checked on the host before any HIP call; on error the
 *   call returns a negative FA_ERR_* code, enqueues nothing and leaves every
 *   output untouched. A failed kernel launch returns FA_ERR_HIP. Empty problems
 *   (B, Hq or N_q equal to 0) return FA_OK and enqueue nothing.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and the 16-bit outputs. fa_dtype is a plain int
 * (not the enum type) so that any value a caller passes is a defined value
 * of the parameter; the library rejects values other than these three with
 * FA_ERR_UNSUPPORTED. */
enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 };
typedef int fa_dtype;

enum {
  FA_OK = 0,
  FA_ERR_NULLPTR = -1,     /* a required pointer is NULL                     */
  FA_ERR_SHAPE = -2,       /* negative size, Hkv == 0 or Hq % Hkv != 0       */
  FA_ERR_UNSUPPORTED = -3, /* d, dtype or pass not supported                 */
  FA_ERR_ALIGNMENT = -4,   /* pointer not 16-byte (workspace: 256) aligned   */
  FA_ERR_WORKSPACE = -5,   /* workspace smaller than fa_*_workspace_size()   */
  FA_ERR_SCALE = -6,       /* scale not finite or not > 0; causal not 0 / 1  */
  FA_ERR_HIP = -7,         /* the HIP runtime reported an error at launch    */
  FA_ERR_OVERLAP = -8,     /* an output overlaps an input                    */
  FA_ERR_SCRATCH = -9      /* needs more than the static scratch (fa_bwd_noalloc) */
};

/* Bytes of device workspace fa_fwd needs for this problem. Zero for prefill
 * (N_q > 1) and for FA_F32; for N_q == 1 with a 16-bit dtype (decode) the
 * key range is split across workgroups and the workspace holds each split's
 * partial row state (O_s, LSE_s), merged with the rescaling rule of [KB] §04.
 * Returns 0 for an invalid or empty problem. */
size_t fa_fwd_workspace_size(int B, int Hq, int Hkv, int Nq, int Nkv, int d, fa_dtype dt);

/* Bytes of device workspace fa_bwd needs: the float32 row terms -D_i
 * (D_i = sum_c dO_ic O_ic) and -LSE_i / scale, each [B, Hq, N_q] (at byte
 * offsets 0 and R = 4 B Hq N_q rounded up to a multiple of 256; -D_i / r
 * with dropout), and, when there are too few key blocks
 * to fill the GPU (e.g. MQA), float32 partial dK and dV sums of the split
 * query-head groups. Linear in N ([KB] §06: storage O(N), not O(N^2)).
 * Returns 0 for an invalid or empty problem. */
size_t fa_bwd_workspace_size(int B, int Hq, int Hkv, int Nq, int Nkv, int d, fa_dtype dt);

/* Forward ([BLOG] §五, [KB] §03-§04): O = softmax(scale * Q K^T + mask) V and
 * the row LSE. Outer loop over query tiles (one workgroup each), inner loop
 * over the key/value tiles the tile may see, folded in with the online
 * softmax update of [KB] §04 (m, l, U rescaled by exp(m_old - m_new)).
 * Reads q, k, v; writes o (input dtype) and lse (float32). */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           void* workspace, size_t workspace_bytes,
           int B, int Hq, int Hkv, int Nq, int Nkv, int d,
           float scale, int causal, fa_dtype dt, hipStream_t stream);

/* Backward ([KB] §05; [NEWS]): given the forward's inputs, its output o and
 * lse, and the output gradient dO, recompute each probability tile
 * P = exp(scale * Q K^T - LSE) and produce dq, dk, dv (input dtype):
 *   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D_i = sum_c dO_ic O_ic,
 *   dQ = scale dS K,  dK = scale dS^T Q,
 * with dK, dV of a key/value head summed over the query heads that read it.
 * FA_F16 and FA_BF16 only. Runs the three stages of fa_bwd_stage in order. */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dO, void* dq, void* dk, void* dv,
           void* workspace, size_t workspace_bytes,
           int B, int Hq, int Hkv, int Nq, int Nkv, int d,
           float scale, int causal, fa_dtype dt, hipStream_t stream);

/* One stage of fa_bwd, same arguments, for callers that interleave or time
 * the stages. Stages must run in order 0, 1, 2 on one workspace:
 *   0  per query tile: recompute P and dS over the key/value tiles it sees
 *      and write dq; store the row terms -D_i and -LSE_i / scale into the
 *      workspace;
 *   1  per key/value block: recompute P and dS over the query tiles that see
 *      it (from stage 0's row terms) and write dk, dv (float32 partials into
 *      the workspace when the query-head group is split);
 *   2  add up split dk, dv partials (enqueues nothing when the group is not
 *      split).
 * Any other stage value returns FA_ERR_UNSUPPORTED. */
int fa_bwd_stage(int stage,
                 const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dO, void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes,
                 int B, int Hq, int Hkv, int Nq, int Nkv, int d,
                 float scale, int causal, fa_dtype dt, hipStream_t stream);

/* fa_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops that must not call hipMalloc, harnesses that
 * forbid allocation). The same computation as fa_bwd, with the same
 * arguments except the workspace: the library uses its own static device
 * buffer of FA_NOALLOC_SCRATCH_BYTES bytes per GPU instead, which exists
 * from the first call on a device until the process ends. Nothing is
 * allocated or freed by the call (the buffer's address is looked up once
 * per device, on that device's first call, under a lock).
 * Limit: problems whose fa_bwd_workspace_size exceeds
 * FA_NOALLOC_SCRATCH_BYTES return FA_ERR_SCRATCH and enqueue nothing.
 * Every call on one GPU uses that GPU's one buffer, and the stages of a
 * call rewrite what they read from it before reading it, so nothing needs
 * clearing between calls; but two calls that overlap in time on one GPU
 * (different streams, or host threads enqueuing concurrently) race on the
 * buffer and must be ordered by the caller. Status codes and execution as
 * fa_bwd, plus FA_ERR_SCRATCH, and FA_ERR_HIP when the buffer's address
 * cannot be obtained. */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dO, void* dq, void* dk, void* dv,
                   int B, int Hq, int Hkv, int Nq, int Nkv, int d,
                   float scale, int causal, fa_dtype dt, hipStream_t stream);

/* Decode (one query row per sequence) over a paged K/V cache ([KB]
 * "FlashAttention：为什么少搬数据，反而算得更快" §09 names paged KV as the
 * decode-side neighbour of FlashAttention; this is the same split-KV decode as
 * fa_fwd with N_q == 1, its K/V gathered through a page table):
 *   q          [B, Hq, 1, d], dtype dt (FA_F16 or FA_BF16)
 *   k_pages,   [num_pages, Hkv, page_size, d] page pools, dtype dt: page n
 *   v_pages    holds, for every kv head, page_size consecutive keys
 *   page_table int32 [B, max_pages], device memory: entry p of row b is the
 *              pool page that holds keys p*page_size .. (p+1)*page_size - 1
 *              of sequence b
 *   seq_lens   int32 [B], device memory: keys of sequence b (the query row
 *              sees all of them; causal masking has no effect with one row)
 *   o          [B, Hq, 1, d], dtype dt;  lse [B, Hq] float32
 * page_size must be a positive multiple of 64. Values in device memory are
 * not checked on the host: a table entry outside [0, num_pages) names no
 * page, and the keys it would hold are dropped from the attention (never
 * read, never scored); lengths are clamped to [0, max_pages * page_size]. A
 * sequence of length 0, or whose every entry is out of range, gets o = 0,
 * lse = -inf. Entries past a sequence's last page are not read. The workspace (fa_fwd_paged_workspace_size) holds the
 * float32 partial results of the key-range splits; 256-byte aligned. Same
 * status codes and aliasing rules as fa_fwd; asynchronous on stream. */
int fa_fwd_paged(const void* q, const void* k_pages, const void* v_pages,
                 const int* page_table, const int* seq_lens, void* o, float* lse,
                 void* workspace, size_t workspace_bytes,
                 int B, int Hq, int Hkv, int num_pages, int page_size, int max_pages, int d,
                 float scale, fa_dtype dt, hipStream_t stream);

/* Bytes of device workspace fa_fwd_paged needs (0 for an invalid or empty
 * problem). */
size_t fa_fwd_paged_workspace_size(int B, int Hq, int Hkv, int page_size, int max_pages, int d,
                                   fa_dtype dt);

/* Dropout on the attention probabilities ([KB] §04 lists dropout among what
 * the tiled computation must still get right; [KB] §08's example call carries
 * a dropout probability). Inverted dropout on the normalised P, with keep
 * mask Z:
 *   O = r (P o Z) V,  r = 256 / (256 - theta),  theta = min(255, floor(256 p + 1/2)),
 * and lse exactly as fa_fwd (the mask does not enter it). Like P ([KB] §05)
 * the mask is never stored: element (b, h, i, j) -- query head h, query row
 * i, key j -- is kept iff byte t = j mod 32 of the 256-bit block of the
 * counter-based generator Philox4x64-10 (Salmon, Moraes, Dror, Shaw,
 * "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011) for counter
 * (floor(j / 32), i, b * Hq + h, offset) and key (seed, 0) is >= theta, byte
 * t being bits 8 (t mod 8) .. +7 of output word floor(t / 8). A caller draws
 * a fresh mask by changing seed or offset; the backward (fa_bwd_dropout) of
 * one forward must use the same (dropout_p, seed, offset).
 * dropout_p: finite, 0 <= p < 1 (else FA_ERR_SCALE); p = 0 gives fa_fwd's
 * result. FA_F16 and FA_BF16 only (FA_F32: FA_ERR_UNSUPPORTED). All other
 * arguments, the workspace (size from fa_fwd_workspace_size) and the status
 * codes are those of fa_fwd; asynchronous on stream. */
int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                   void* workspace, size_t workspace_bytes,
                   int B, int Hq, int Hkv, int Nq, int Nkv, int d,
                   float scale, int causal, float dropout_p, uint64_t seed, uint64_t offset,
                   fa_dtype dt, hipStream_t stream);

/* Backward of fa_fwd_dropout, for the same (dropout_p, seed, offset): the
 * keep mask is drawn again, tile by tile, exactly as the forward drew it, and
 * with r and Z as above
 *   dV = r (P o Z)^T dO,  dP = r Z o (dO V^T),  dS = P * (dP - D),
 *   D_i = sum_c dO_ic O_ic (still equal to sum_j P_ij dP_ij),
 *   dQ = scale dS K,  dK = scale dS^T Q.
 * o and lse are fa_fwd_dropout's outputs. dropout_p: finite, 0 <= p < 1
 * (else FA_ERR_SCALE). Otherwise the arguments, workspace (size from
 * fa_bwd_workspace_size) and status codes are those of fa_bwd. */
int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dO, void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes,
                   int B, int Hq, int Hkv, int Nq, int Nkv, int d,
                   float scale, int causal, float dropout_p, uint64_t seed, uint64_t offset,
                   fa_dtype dt, hipStream_t stream);

/* The keep mask Z of fa_fwd_dropout for the same (dropout_p, seed, offset),
 * written out as bytes: keep [B, Hq, N_q, N_kv] uint8 in device memory, 1 =
 * kept, 0 = dropped, every byte written (also where the causal mask hides the
 * key). For tests and debugging: the attention calls draw the same bits and
 * never write them. No alignment requirement. FA_ERR_SCALE for a bad
 * dropout_p, FA_ERR_SHAPE for a negative size, FA_ERR_UNSUPPORTED when
 * B * Hq >= 2^31; empty sizes return FA_OK. Asynchronous on stream. */
int fa_dropout_mask(unsigned char* keep, int B, int Hq, int Nq, int Nkv, float dropout_p,
                    uint64_t seed, uint64_t offset, hipStream_t stream);

/* FP8 forward ([KB] §07 notes an FP8 path of the same algorithm on Hopper):
 * q [B, Hq, N_q, 128], k, v [B, Hkv, N_kv, 128] hold OCP E4M3 codes (1 byte
 * each: sign, 4 exponent bits with bias 7, 3 mantissa bits; largest finite
 * 448; 0x7F, 0xFF are NaN) whose real values are code value * descale_q
 * (descale_k, descale_v). Computes the attention of those real values with
 * scale and causal as in fa_fwd, using E4M3 operands on the matrix cores for
 * S = Q K^T and for P V, where the probabilities (each taken relative to a
 * running row maximum, so at most 256) are rounded to E4M3 nearest-even;
 * the softmax state and all sums are float32. Writes o [B, Hq, N_q, 128] as
 * bf16 and lse [B, Hq, N_q] float32 (natural log). Head dim 128 only
 * (FA_ERR_UNSUPPORTED otherwise); descale factors finite and > 0 (else
 * FA_ERR_SCALE). No workspace. Alignment, aliasing, status codes and
 * execution as fa_fwd. */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int Nq, int Nkv, int d,
               float scale, int causal, float descale_q, float descale_k, float descale_v,
               hipStream_t stream);

/* Static English text for a status code (never NULL). */
const char* fa_strerror(int status);

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
