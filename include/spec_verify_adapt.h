/*
 * spec_verify_adapt.h -- C ABI of the adaptive draft-length controller and
 * the acceptance statistics that follow each verify step (same library as
 * spec_verify.h).
 *
 * The operation (pages cited by title and section):
 *   [D] "大模型推理加速新范式：推测解码（Speculative Decoding）原理剖析与
 *       vLLM生产级实现", section 4.3: a sliding window of per-step
 *       acceptance ratios drives the draft length K; when the window's mean
 *       is above a band around a target K grows by one, below it K shrinks
 *       by one, within [k_min, k_max]; no change before the window holds a
 *       minimum number of ratios.  Section 4.2: the accept rate
 *       (accepted / drafted) is the core metric to watch.
 *   [B] the blog.hotdry.top post on speculative decoding and dynamic
 *       batching, 延迟权衡与自适应策略 and 工程落地参数清单: adjust the
 *       candidate length from the pass rate of the last 10 rounds, +1 above
 *       80%, -1 below 50%, starting from 4-8.
 *
 * One controller per request slot (a continuous-batching server keeps a
 * request in one slot while it decodes).  After a verify step, for every
 * sequence b of the batch (slot s = slots[b], drafted = gamma_b =
 * cu_draft[b+1] - cu_draft[b], accepted = num_accepted[b]):
 *   alpha = accepted / max(drafted, 1)                      (double)
 *   the slot keeps its last `window` ratios (the oldest drops out);
 *   with at least `min_history` of them, mean = their sum, added
 *   sequentially oldest first in double, divided by their count, and
 *     mean > up   : k = min(k + 1, k_max)
 *     mean < down : k = max(k - 1, k_min)
 *   next_k[b] = the slot's k (the next step's gamma_b), and next_cu = the
 *   exclusive prefix of next_k (the next step's cu_draft, B+1 entries).
 * Statistics (optional, four uint64 the caller clears once and the calls
 * accumulate): sequences verified, drafts accepted, drafts proposed, tokens
 * emitted (accepted + 1 per sequence).  The accept rate of [D] 4.2 is
 * stats[1] / stats[2].
 *
 * Presets (each value as the page prints it; readings in brackets):
 *   SPEC_VERIFY_ADAPT_PRESET_WINDOW50 ([D] 4.3): k in [2, 8], k_init 2,
 *     window 50, min_history 10, up = 0.6 + 0.1, down = 0.6 - 0.1.
 *   SPEC_VERIFY_ADAPT_PRESET_LAST10 ([B]): k in [1, 8] [the lower bound is a
 *     reading], k_init 4, window 10, min_history 10 [a reading: act on full
 *     windows], up 0.8, down 0.5.
 *
 * Memory: `state` is caller-owned, spec_verify_adapt_state_bytes() long,
 * 256-byte aligned, and lives where `device` says: device = -1 means every
 * pointer is host memory and the call computes synchronously on the calling
 * thread; device >= 0 means every pointer is device memory of that device
 * (which must be current) and the call only enqueues work on `hip_stream`.
 * A slot must be reset (spec_verify_adapt_reset) before its first update.
 * Slots must be distinct within one update; updates that share a state must
 * be ordered (same stream, or the same host thread).
 *
 * Errors: OK (0) or a negative spec_verify.h code, checked on the host before
 * any HIP call: EINVAL for bad parameters, NULL required pointers, a batch
 * larger than num_slots without a slot list, a wrong current device;
 * ECAPACITY for a short state buffer; EHIP for a failed launch.  Bad device
 * data is never an out-of-bounds access: a slot outside [0, num_slots) or
 * counts with accepted outside [0, drafted] leave every controller
 * unchanged, report the slot's current k (k_init for a bad slot), are not
 * counted, and set SPEC_VERIFY_ADAPT_BAD_* bits in *status when given.
 */
#ifndef SPEC_VERIFY_ADAPT_H_
#define SPEC_VERIFY_ADAPT_H_

#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_VERIFY_ADAPT_HOST (-1)
#define SPEC_VERIFY_ADAPT_PRESET_WINDOW50 0
#define SPEC_VERIFY_ADAPT_PRESET_LAST10 1
#define SPEC_VERIFY_ADAPT_BAD_SLOT 1u
#define SPEC_VERIFY_ADAPT_BAD_COUNTS 2u
#define SPEC_VERIFY_ADAPT_MAX_WINDOW 4096

typedef struct {
  int32_t k_min;       /* >= 0 */
  int32_t k_max;       /* >= k_min */
  int32_t k_init;      /* in [k_min, k_max] */
  int32_t window;      /* ratios kept, 1 .. SPEC_VERIFY_ADAPT_MAX_WINDOW */
  int32_t min_history; /* ratios needed before a change, 1 .. window */
  int32_t reserved;    /* 0 */
  double up;           /* mean > up grows k (finite) */
  double down;         /* mean < down shrinks k (finite, <= up) */
} spec_verify_adapt_params;

/* Fill *out with a preset.  Returns OK or EINVAL. */
SPEC_VERIFY_API int spec_verify_adapt_preset(int which, spec_verify_adapt_params *out);

/* Bytes of state for num_slots controllers with these parameters (host only,
 * no HIP call).  Returns OK or EINVAL. */
SPEC_VERIFY_API int spec_verify_adapt_state_bytes(const spec_verify_adapt_params *params,
                                                  int64_t num_slots, size_t *bytes);

/* Reset `count` slots (slots[0..count), or every slot when slots is NULL)
 * to k_init with an empty history. */
SPEC_VERIFY_API int spec_verify_adapt_reset(const spec_verify_adapt_params *params,
                                            int64_t num_slots, void *state,
                                            size_t state_bytes, int64_t count,
                                            const int32_t *slots, int device,
                                            void *hip_stream);

/* One step for a batch of num_seqs sequences (slots NULL: sequence b uses
 * slot b).  cu_draft [B+1] and num_accepted [B] are a verify call's input
 * offsets and output counts; next_k [B] is written; next_cu [B+1], stats [4]
 * and status [1] are optional. */
SPEC_VERIFY_API int spec_verify_adapt_update(const spec_verify_adapt_params *params,
                                             int64_t num_slots, void *state,
                                             size_t state_bytes, int32_t num_seqs,
                                             const int32_t *slots, const int32_t *cu_draft,
                                             const int32_t *num_accepted, int32_t *next_k,
                                             int32_t *next_cu, uint64_t *stats,
                                             uint32_t *status, int device,
                                             void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_ADAPT_H_ */
