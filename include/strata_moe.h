/*
 * strata_moe.h — C ABI of one routed 4-bit Mixture-of-Experts FFN layer that
 * runs under an expert budget on an AMD Instinct MI355X (gfx950).
 *
 * What the layer computes (the forward of one MoE FFN block):
 *   router logits l = x Wr^T (+ b), top-k experts per token, routing weights
 *   (softmax over the selected logits, or sigmoid renormalised over them),
 *   tokens grouped by expert, per expert a SwiGLU FFN o = Wd (silu(Wg x) * Wu x)
 *   computed straight from 4-bit packed weights, and y = sum_j w_j o_j (+ the
 *   shared expert's output).
 *
 * Sources (page title, section):
 *   - "Documentation" (strata.amperor.ai docs), Signature: a model loads with
 *     a budget of resident experts per layer (or a RAM target that implies
 *     one) and a paging policy; the rest of the experts are streamed.
 *   - "Strata, Explained" (Medium tutorial), section 2: GPU memory holds the
 *     router, the shared experts and a cache of the most-used experts that
 *     adapts to the workload, host RAM holds every expert pinned; a 512-expert
 *     layer activates 10 routed experts plus 1 shared expert per token.
 *   - ro99/strata README (C++20/CUDA engine): its list of enforced rules
 *     (weights stay at four bits or more; the router's arithmetic, the expert
 *     count and k are the checkpoint's, unchanged; prediction may change the
 *     order of work, not its numbers; a configuration that cannot be served
 *     exactly is an error, not a cheaper substitute); precision paragraph (MXFP4 = two E2M1
 *     codes per byte and one E8M0 exponent per 32, read as stored with no
 *     wider copy; E8M0 bytes 0 and 255 fail admission at load); SM86 kernel
 *     paragraph (a prepack of the 4-bit weights into kernel operand order is a
 *     pure permutation of the same byte count).
 *
 * Conventions of every entry point:
 *   - Return a strata_status; on failure the thread-local message returned by
 *     strata_last_error() says why.  Nothing falls back to a different
 *     computation: an unsupported configuration is an error.
 *   - "device pointer" means memory of the GPU the handle was created on;
 *     "host pointer" means ordinary CPU memory.
 *   - A handle is not thread-safe; one thread at a time may use it.
 */
#ifndef STRATA_MOE_H
#define STRATA_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct strata_moe strata_moe; /* opaque; owned by the library */

typedef enum {
  STRATA_OK = 0,
  STRATA_E_INVALID = 1,     /* null pointer, size out of range, bad enum       */
  STRATA_E_UNSUPPORTED = 2, /* shape or value the kernels cannot take exactly  */
  STRATA_E_BAD_SCALE = 3,   /* admission: MXFP4 E8M0 byte 0 or 255, NVFP4 E4M3 NaN byte or matrix scale
                             * not finite and > 0, int4 scale or bias NaN or infinite */
  STRATA_E_NOMEM = 4,       /* host-pinned or device allocation failed         */
  STRATA_E_HIP = 5,         /* a HIP runtime call failed                       */
  STRATA_E_POISONED = 6     /* an earlier HIP failure left the handle unusable */
} strata_status;

/* 4-bit expert weight formats. */
typedef enum {
  /* int4 codes, one bf16 scale s and one bf16 bias b per 64 consecutive inputs
   * of a row: w = s * q + b, q in 0..15 (the MLX-style "4bit" affine form). */
  STRATA_Q_INT4_G64_AFFINE_BF16 = 1,
  /* OCP MXFP4: E2M1 codes (sign bit 3), one E8M0 exponent byte e per 32
   * consecutive inputs of a row: w = e2m1(code) * 2^(e - 127), e in 1..254. */
  STRATA_Q_MXFP4_E2M1_E8M0_G32 = 2,
  /* int4 affine as above with one (s, b) per 128 consecutive inputs (the
   * "INT4 group-128, W4A16" of the ro99/strata README model table). */
  STRATA_Q_INT4_G128_AFFINE_BF16 = 3,
  /* NVFP4 (named in the same table; the published format): E2M1 codes, one
   * OCP FP8 E4M3 scale byte per 16 consecutive inputs of a row and one fp32
   * scale g per matrix: w = e2m1(code) * e4m3(byte) * g.  E4M3 NaN bytes
   * (0x7F, 0xFF) fail admission. */
  STRATA_Q_NVFP4_E2M1_E4M3_G16 = 4
} strata_quant;

typedef enum {
  /* softmax over the k selected logits (equals softmax over all experts
   * renormalised to the top k) */
  STRATA_R_SOFTMAX_TOPK_RENORM = 1,
  /* sigmoid of each selected logit divided by the sum over the k selected */
  STRATA_R_SIGMOID_TOPK_RENORM = 2
} strata_router;

/* Residency policies.  The pages name policies (none, warm, cache, hybrid) on
 * the "Documentation" page (Signature) without defining them, say the GPU
 * cache adapts to the workload ("Strata, Explained", section 2) at a rate that
 * is tuned per machine and that its learned state can be saved, one profile
 * per kind of work (same page, section 8).  Every expert carries a frequency
 * score (one use = 65536; see strata_expert_profile_save).  A policy only
 * decides what is paged and when; it never changes y. */
typedef enum {
  STRATA_P_LRU = 1, /* evict the least recently used, ties to the lower id */
  STRATA_P_LFU = 2, /* evict the lowest score, then least recent, then lower id */
  STRATA_P_WARM = 3 /* LFU order on a decaying score: after every forward each
                     * score loses score >> decay_shift before the uses of that
                     * forward are added, so old use fades at 1 - 2^-decay_shift
                     * per forward (the cache's adaptation rate) */
} strata_policy;

/* How missing experts travel from the pinned host store into HBM slots.
 * KERNEL: the library's page-in kernel reads the store through its device
 * mapping (64 small workgroups; in a prefill on 16 CUs set aside for paging,
 * two per XCD, the copy streams' CU mask, while the layer's expert kernels of
 * that forward run on an internal stream masked to the other CUs; in a decode
 * forward on the caller's stream, before its expert kernels).  DMA: one
 * hipMemcpyAsync per record on the copy streams (the DMA engines; no CU
 * time, but the HIP runtime held the host 5-15 ms inside single copy calls
 * now and then on layers with small records).  AUTO: KERNEL for records of
 * at most 8 MiB, DMA above (measured: equal mean on small records without the
 * stalls, 1-3% slower than DMA on records of 9 MB and more).  Only the paging
 * engine differs; y is the same. */
typedef enum {
  STRATA_PAGER_AUTO = 0,
  STRATA_PAGER_KERNEL = 1,
  STRATA_PAGER_DMA = 2
} strata_pager;

/* One stacked packed matrix, host pointers, row-major [out, in] per expert and
 * quantised along `in`.  Element 2i of a row is the low nibble of byte i.
 *   codes  : u8   [n_exp, out, in/2]
 *   scales : int4 -> bf16 bits [n_exp, out, in/G] (G = 64 or 128);
 *            MXFP4 -> u8 E8M0 [n_exp, out, in/32]; NVFP4 -> u8 E4M3 [n_exp, out, in/16]
 *   biases : int4 -> bf16 bits [n_exp, out, in/G]; MXFP4, NVFP4 -> must be NULL
 *   global_scale : NVFP4 -> fp32 [n_exp], each finite and > 0; others -> must be NULL
 * Gate and up are [F, H] (out = F, in = H); down is [H, F]. */
typedef struct {
  const void* codes;
  const void* scales;
  const void* biases;
  const float* global_scale;
} strata_qmat;

typedef struct {
  int32_t hidden;        /* H: multiple of 512                               */
  int32_t ffn;           /* F: multiple of 64 (128 for int4 group-128)       */
  int32_t num_experts;   /* E: routed experts, 1..1024                       */
  int32_t top_k;         /* k: 1..min(E, 32)                                 */
  int32_t num_shared;    /* 0 or 1 shared expert (weight 1, always resident) */
  int32_t quant;         /* strata_quant                                     */
  int32_t router;        /* strata_router                                    */
  int32_t policy;        /* strata_policy                                    */
  int32_t expert_budget; /* resident routed experts (HBM slots), 1..E         */
  int32_t max_tokens;    /* largest T a forward may take (sizes the workspace) */
  int32_t device;        /* HIP device ordinal; -1 = the current device       */
  int32_t decay_shift;   /* WARM: 1..24; other policies: must be 0            */
  int32_t prefetch;      /* 0..budget: most experts paged ahead after a forward
                          * (non-residents that outrank a resident under the
                          * policy's order, hottest first, into the coldest
                          * residents' slots); 0 = off                        */
  int32_t pager;         /* strata_pager                                     */
  const uint64_t* expert_profile; /* host [E] scores (each <= 2^62) to warm the
                          * slots with at create, or NULL (see
                          * strata_expert_profile_load)                       */
  const uint16_t* router_w;   /* host, bf16 bits [E, H]                        */
  const float* router_bias;   /* host, fp32 [E], or NULL                       */
  strata_qmat gate, up, down; /* routed experts, n_exp = E                     */
  strata_qmat sh_gate, sh_up, sh_down; /* shared expert, n_exp = 1, or all NULL */
  /* Shared-expert gate: host, bf16 bits [H], or NULL.  With it (num_shared
   * must be 1) the shared expert's output is weighted by sigmoid(l_s) per
   * token, l_s = x . w_s formed in fp32 in the router's summation order;
   * without it the weight is 1.  The ro99/strata README's model table lists
   * shared experts beside routed ones without saying how they are weighted;
   * both forms are offered. */
  const uint16_t* shared_gate_w;
  /* Hybrid decode (the "Documentation" page's policy value hybrid; "Strata,
   * Explained", section 2: the host computes the experts the GPU does not
   * hold, at the same time): 0 = off; 1 = in a decode forward (T <= 8) of a
   * budgeted layer, the experts resident at call start run on the GPU and
   * every other needed expert is computed by host threads from the pinned
   * store (fp32, each output row summed by one thread in a fixed order), with
   * no page made for it; scores and prefetch (desc.prefetch) are updated as
   * in any forward, so the cache still adapts.  y is then within the layer's
   * tolerance of the all-resident y, not bitwise equal to it.  Prefill
   * forwards page as usual unless hybrid_rows is set. */
  int32_t hybrid;
  int32_t host_threads; /* hybrid: host threads computing experts (the
                         * calling thread is one of them); 0 = the CPUs this
                         * process may run on */
  /* Hybrid prefill (hybrid = 1 only): 0 = off; R in 1..8 = in a forward of
   * more than 8 tokens of a budgeted layer, a needed expert that is not
   * resident at call start and has at most R tokens is computed by the host
   * threads (as above) instead of being paged, while the GPU runs and pages
   * the others; scores and prefetch cover every needed expert.  Few-token
   * experts cost the host little arithmetic but a whole record over the
   * link, so the host takes part of the link's load. */
  int32_t hybrid_rows;
} strata_moe_desc;

/* Creates a layer.  Validates the descriptor, admits the weights (every MXFP4
 * scale byte must be in 1..254, every NVFP4 E4M3 byte a number and every
 * NVFP4 matrix scale finite and > 0, every int4 scale and bias a finite
 * bf16 number; int4 layers run in fp16, so each matrix's scales and biases
 * are stored times one power of two that makes them exact fp16 numbers, and
 * a matrix whose values span more than fp16 holds exactly under one such
 * power of two, about 2^-24 .. 2^15 relative to each other, is refused with
 * E_UNSUPPORTED), copies every routed
 * expert once into a library-owned pinned host store (a byte permutation into
 * kernel tile order: same byte count, no wider copy), allocates the HBM slot
 * pool (expert_budget slots), the resident shared expert, the router and a
 * workspace sized by max_tokens, and preloads routed experts 0..budget-1 into
 * slots 0..budget-1, or, given expert_profile, the budget experts with the
 * largest scores (ties to the lower id; those among 0..budget-1 keep their
 * slots, the rest fill the freed slots in ascending id order).  The caller's
 * buffers may be freed when this returns.
 * Errors: E_INVALID, E_UNSUPPORTED, E_BAD_SCALE, E_NOMEM, E_HIP.  On error
 * *out is NULL and nothing is leaked. */
strata_status strata_moe_create(const strata_moe_desc* desc, strata_moe** out);

/* Optional routing outputs of a forward, device pointers, each may be NULL.
 *   logits  fp32 [T, E]       router logits
 *   topk_idx int32 [T, k]     selected experts, rank order
 *   topk_w  fp32 [T, k]       routing weights
 *   counts  int32 [E]         tokens per expert
 *   offsets int32 [E + 1]     exclusive prefix sum of counts
 *   perm    int32 [T * k]     token ids grouped by expert, ascending inside one */
typedef struct {
  float* logits;
  int32_t* topk_idx;
  float* topk_w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
} strata_route_dbg;

/* One forward of the layer on T tokens.
 *   x      device, bf16 bits [T, H] row-major, caller-owned, read only; any
 *          finite bf16 values (int4 and NVFP4 layers compute in fp16 and
 *          rescale every token row, and the SwiGLU output, by powers of two,
 *          so neither overflows nor flushes; elements below 2^-32 of their
 *          row's largest magnitude round to that row's fp16 grid)
 *   y      device, bf16 bits [T, H] row-major, caller-owned, written (RNE)
 *   stream hipStream_t to enqueue on (NULL = the null stream)
 *   dbg    optional routing outputs (NULL = none)
 * x and y must not overlap.  The call enqueues its work on `stream`.  When the
 * budget is smaller than E it waits once for the per-expert token counts to
 * reach the host, decides hits and misses, and pages missing experts from the
 * pinned store into slots (by the engine desc->pager chose): a prefill pages on
 * internal copy streams and runs the expert kernels on an internal compute
 * stream (ordered after the routing on `stream`, and the combine on `stream`
 * after it); a decode forward (T <= 8) with the page-in kernel pages and
 * computes on `stream` itself, and one that pages nothing computes there; if
 * more distinct experts are needed than there are slots, the policy's
 * hottest quarter of the slots stays put and the experts stream through the
 * rest in waves of half of it, so one wave's pages land while the previous
 * wave computes.  Paging, waves and slot placement never change y (it is
 * bitwise the same as with budget = E).  T == 0 is a no-op.
 * Graph capture: a forward of a layer whose budget is E (all experts
 * resident) enqueues only kernels, so it may be captured into a HIP graph on
 * `stream` and replayed; a replay computes from whatever x holds then.  Replays
 * share the layer's workspace with every other forward of the layer, so the
 * caller orders them (one stream); the statistics count the captured forward
 * once, not its replays.  A budgeted forward decides its pages on the host and
 * cannot be captured (E_UNSUPPORTED), nor can a forward with kernel timing on.
 * Errors: E_INVALID (null handle or pointers, T < 0, T > max_tokens),
 * E_UNSUPPORTED (capture, above), E_HIP (after which the handle is poisoned),
 * E_POISONED. */
strata_status strata_moe_forward(strata_moe* h, const void* x, int32_t T, void* y, void* stream,
                                 const strata_route_dbg* dbg);

/* No-allocation forward, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, semantics and result as strata_moe_forward
 * (bitwise the same y and routing outputs), except that the forward's device
 * buffers (logits, routing lists, h, o, the scaled fp16 copy of x) come from
 * a static scratch array inside the library instead of the handle's
 * workspace, and the call allocates nothing.  The array is 64 MiB, one copy
 * per GPU, held until the process ends; its address on a device is looked up
 * when the first layer is created there.  T may exceed neither max_tokens
 * nor the largest T whose buffers fit 64 MiB (about T * (4 E + R (2 F +
 * 4 H P) + 2 H) bytes with R = k + num_shared rows per token and P the
 * prefill down GEMM's partial-sum planes; E_INVALID names that T).  Every
 * call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (different streams, or different layers without ordering between them)
 * race; calls on one stream are ordered.  The array keeps what the last call
 * left in it; no part needs clearing, since a forward writes every element
 * before reading it.  Requires budget == E (a budgeted forward plans its
 * pages in host memory that it allocates: E_UNSUPPORTED) and kernel timing
 * off (E_UNSUPPORTED).  Errors: as strata_moe_forward. */
strata_status strata_moe_forward_noalloc(strata_moe* h, const void* x, int32_t T, void* y, void* stream,
                                         const strata_route_dbg* dbg);

/* Cumulative counters since create ("/health" style live state: policy,
 * budget, resident bytes). */
typedef struct {
  uint64_t forwards;       /* forwards with T > 0                              */
  uint64_t hits;           /* needed experts already resident at call start    */
  uint64_t misses;         /* needed experts paged in                          */
  uint64_t evictions;      /* pages that overwrote a resident expert           */
  uint64_t bytes_h2d;      /* expert bytes paged host -> device                */
  uint64_t waves;          /* expert waves run                                 */
  int32_t budget;          /* slots                                            */
  int32_t resident;        /* slots holding an expert                          */
  int32_t policy;          /* strata_policy                                    */
  int32_t decay_shift;     /* as created                                       */
  uint64_t resident_bytes; /* resident * expert_bytes                          */
  uint64_t expert_bytes;   /* packed bytes of one expert                       */
  uint64_t prefetched;     /* experts paged ahead of need (prefetch, run-time
                            * profile loads); included in bytes_h2d and, when
                            * they overwrote an expert, in evictions           */
  uint64_t prefetch_hits;  /* hits on an expert paged ahead, first use only    */
  int32_t prefetch;        /* as created                                       */
  int32_t pager;           /* the paging engine in use (KERNEL or DMA; 0 in a
                            * residency replay)                                */
  uint64_t host_experts;   /* hybrid: needed experts computed on the host      */
  uint64_t host_ns;        /* hybrid: wall time of those host computations     */
} strata_cache_stats;

/* Reads the counters.  Does no device work except, when budget == E, one
 * blocking read of a device-side counter of distinct experts used.
 * Errors: E_INVALID (null pointers), E_HIP. */
strata_status strata_expert_cache_stats(const strata_moe* h, strata_cache_stats* out);

/* Device and pinned-host bytes held by a handle.  None of the device terms
 * grows with E * H * F except through the budget: no dequantised copy exists. */
typedef struct {
  uint64_t slot_pool;   /* expert_budget * slot stride                          */
  uint64_t shared;      /* the resident shared expert (0 if none)               */
  uint64_t router;      /* router weights and bias                              */
  uint64_t workspace;   /* activations, routing buffers, outputs for max_tokens */
  uint64_t device_total;
  uint64_t host_store;  /* pinned host bytes of the routed expert store: E
                         * records, each at the 256-byte aligned slot stride */
} strata_memory_info;

strata_status strata_moe_memory(const strata_moe* h, strata_memory_info* out);

/* Kernel timing.  While enabled, every kernel launch of a forward is bracketed
 * by HIP events on the forward's stream; strata_moe_timing() waits for them
 * and returns totals per kernel class, and resets them. */
typedef enum {
  STRATA_K_ROUTER = 0,   /* router logits (T * E <= 1024: and the whole grouping,  */
                         /* done by the launch's last workgroup)                   */
  STRATA_K_GROUP = 1,    /* top-k, weights, counts, offsets, perm, tile list       */
  STRATA_K_DEC_UP = 2,   /* decode gate+up GEMV + SwiGLU                           */
  STRATA_K_DEC_DOWN = 3, /* decode down GEMV                                       */
  STRATA_K_PRE_UP = 4,   /* prefill gate+up grouped GEMM                           */
  STRATA_K_PRE_DOWN = 5, /* prefill down grouped GEMM                              */
  STRATA_K_COMBINE = 6,  /* weighted top-k + shared combine                        */
  STRATA_K_COUNT = 7
} strata_kernel_class;

typedef struct {
  double ms[STRATA_K_COUNT];         /* summed event time per class */
  uint64_t launches[STRATA_K_COUNT]; /* launches per class          */
} strata_timing;

strata_status strata_moe_set_timing(strata_moe* h, int32_t enable);
strata_status strata_moe_timing(strata_moe* h, strata_timing* out);

/* Frees everything the handle owns (waits for its outstanding work first).
 * NULL is ignored. */
void strata_moe_destroy(strata_moe* h);

/* Message of the last failure on this thread ("" if none).  Owned by the
 * library; valid until the next call on this thread. */
const char* strata_last_error(void);

/* Measures the pinned host -> device copy rate of the paging link: allocates
 * `bytes` of pinned host memory and of device memory on `device`, times `iters`
 * hipMemcpyAsync copies with HIP events, frees both and writes GB/s (1e9 B/s).
 * Errors: E_INVALID (bytes == 0, iters < 1, NULL out), E_NOMEM, E_HIP. */
strata_status strata_measure_h2d(int32_t device, uint64_t bytes, int32_t iters, double* gbps);

/* Measures the HBM read ceiling that decode bandwidth is compared with (the
 * "measured read ceiling" of the SM86 kernel paragraph of the ro99/strata
 * README): allocates `bytes` of device memory on `device` (at least 64 MiB;
 * use well over the 256 MB last-level cache so every pass streams from HBM),
 * fills it, then times `iters` passes of a streaming-read kernel (each
 * workgroup reads its own contiguous share with non-temporal 16-byte loads)
 * with HIP events, frees it and writes the best pass in GB/s (1e9 B/s).
 * Errors: E_INVALID (bytes < 64 MiB, iters < 1, NULL out), E_NOMEM, E_HIP. */
strata_status strata_measure_hbm_read(int32_t device, uint64_t bytes, int32_t iters, double* gbps);

/* The learned cache state ("expert_profile_save", "Strata, Explained",
 * section 8): writes the E frequency scores of the layer to `scores` (host,
 * uint64 [num_experts]; one use = 65536, decayed under WARM).  Feeding them
 * back at create (desc.expert_profile) or to strata_expert_profile_load
 * starts a layer warm.  Host only.  Errors: E_INVALID (null pointers,
 * num_experts != E). */
strata_status strata_expert_profile_save(const strata_moe* h, uint64_t* scores, int32_t num_experts);

/* Loads a saved profile into a live layer: sets the scores, then pages the B
 * experts with the largest scores (ties to the lower id) that are not yet
 * resident into the slots of the residents outside that set, on the copy
 * streams, after the previous forward's compute; the next forward waits for
 * them.  Returns without waiting.  Counted as prefetches.  With budget == E it
 * only sets the scores.  Errors: E_INVALID (null pointers, num_experts != E,
 * a score above 2^62), E_HIP (poisons the handle), E_POISONED. */
strata_status strata_expert_profile_load(strata_moe* h, const uint64_t* scores, int32_t num_experts);

/* Dry-run planner (host only, touches no GPU): replays the residency policy of
 * a layer with E experts and `budget` slots over a trace of forwards and
 * reports what a real run would page, the placement-plan side of the budget
 * decision.  policy, decay_shift, prefetch and profile (NULL or E scores
 * applied at create) mean what they mean in strata_moe_desc.  needed_flat
 * holds the needed expert ids of every forward back to back, needed_len[i] of
 * them for forward i (any order, duplicates ignored).  hybrid_flags (NULL =
 * none) marks the forwards that are hybrid decode forwards (see
 * strata_moe_desc.hybrid).  host_rows (0..8) replays the other forwards as
 * hybrid prefills with that row limit (strata_moe_desc.hybrid_rows); then
 * needed_rows (parallel to needed_flat, each >= 1; a duplicate id keeps its
 * first count) gives each needed expert's token count.  If plan_slots is not
 * NULL it receives, per forward and per needed expert in the order the
 * forward runs them (hits ascending, then misses by increasing key, the
 * coldest first; a hybrid decode forward: ascending id; a hybrid prefill:
 * that order, then its host experts ascending), the slot used (-1: computed
 * on the host);
 * its length must be sum(needed_len).  If scores_out is not NULL it receives
 * the E final scores.  Errors: E_INVALID. */
strata_status strata_residency_replay(int32_t num_experts, int32_t budget, int32_t policy,
                                      int32_t decay_shift, int32_t prefetch, const uint64_t* profile,
                                      uint64_t expert_bytes, int32_t n_forwards,
                                      const int32_t* needed_len, const int32_t* needed_flat,
                                      const int32_t* hybrid_flags, const int32_t* needed_rows,
                                      int32_t host_rows, int32_t* plan_slots, uint64_t* scores_out,
                                      strata_cache_stats* out);

#ifdef __cplusplus
}
#endif
#endif /* STRATA_MOE_H */
