/*
 * ditango.h -- C ABI of the MI355X (gfx950) library for partitioned softmax
 * attention with selective attention-state reuse across denoising steps.
 *
 * Source of the method: "DiTango: Cost-Effective Parallel Diffusion
 * Generation with Selective Attention State Reuse" (the DiTango page).
 *
 *   - A DiT layer's 3D-flattened token sequence of N tokens is cut into P
 *     contiguous partitions of S = ceil(N/P) tokens (the last one may be
 *     shorter); sequence-wise partitioning as in Ring-CP (introduction).
 *   - For a (query partition q, KV partition k) pair, the attention state is
 *     (OUT, LSE) per query row (attention-state section): with scaled scores
 *     z_j = scale * q.k_j over the keys j of partition k,
 *         LSE = log sum_j exp(z_j)              (natural log)
 *         OUT = sum_j exp(z_j - LSE) * v_j      (normalised within the pair)
 *   - Each step, every pair is either computed fresh (COMPUTE) or reused from
 *     the state cache (REUSE), per a P x P selection mask (state selection
 *     section; the Fig. 6 example).  t_c is the last step a pair was computed.
 *   - The final output of a row is the composition (Eq. 4) of its P states:
 *         LSE = log sum_k exp(LSE_k),   OUT = sum_k exp(LSE_k - LSE) * OUT_k.
 *
 * Conventions shared by every call:
 *   - All device buffers are allocated and owned by the caller; the library
 *     allocates no device memory, keeps no global state besides a
 *     thread-local error string, and never synchronises the stream.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it and the call returns.
 *   - Q, K, V are bfloat16, laid out [H][N][d] contiguous, in device memory.
 *   - Cached states keep LSE in fp32 and OUT in fp32 (the default) or, when
 *     the shape asks for it (state_dtype = DITANGO_STATE_BF16), in bfloat16
 *     (the bit pattern, rounded to nearest even from the fp32 result), which
 *     halves the cache and the bytes the composition reads; the composed
 *     outputs the merges write are fp32 either way.
 *   - The mask is a host array uint8 [P][P] (row = query partition q, column
 *     = KV partition k); 1 = COMPUTE (fresh), 0 = REUSE.
 *   - Return value: DITANGO_OK (0) or a negative code; the message of the
 *     last failure on the calling thread is ditango_last_error().
 *   - One ditango_states_t must not be used by two threads at once.
 */
#ifndef DITANGO_H
#define DITANGO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DITANGO_OK        0
#define DITANGO_EINVAL   (-1)  /* bad argument: null pointer, bad shape, bad mask   */
#define DITANGO_ENOCACHE (-2)  /* a pair marked REUSE has never been computed       */
#define DITANGO_EHIP     (-3)  /* a HIP runtime call or kernel launch failed        */

#define DITANGO_MAX_P 32       /* largest partition count                             */

#define DITANGO_STATE_F32  0  /* cached OUT in fp32 (4 bytes per element)            */
#define DITANGO_STATE_BF16 1  /* cached OUT in bfloat16 (2 bytes per element)        */

/* Shape of one attention layer.  d must be 64, 72 or 128; 1 <= P <= 32;
 * every partition must be non-empty (P * ceil(N/P) - N < ceil(N/P)). */
typedef struct {
  int32_t H;      /* attention heads                                   */
  int32_t N;      /* tokens in the flattened sequence; N * d < 2^30    */
  int32_t d;      /* head dimension                                    */
  int32_t P;      /* partitions                                        */
  float   scale;  /* score scale applied to q.k, normally 1/sqrt(d)    */
  int32_t state_dtype;  /* DITANGO_STATE_F32 (0) or DITANGO_STATE_BF16 (1): cached OUT */
} ditango_shape_t;

/* The attention-state cache (attention-state section and the
 * ring-based composed attention section: fresh states are stored for
 * reuse at later steps).  One slot per (head, pair), pair id = q*P + k:
 *   O   device [H][P*P][S][d]       -- fp32 or bf16 (shape.state_dtype); row r
 *                                     of slot (h, q*P+k) is OUT of
 *                                     query row q*S + r against partition k
 *   LSE device fp32 [H][P*P][S]     -- its log-sum-exp
 *   tc  host int32 [P*P]            -- step at which the pair was last fresh,
 *                                     -1 if never (t_c of the state-selection
 *                                     section)
 * Rows at or beyond the length of a ragged last partition are never written
 * or read.  The struct borrows the three buffers; the caller frees them. */
typedef struct {
  ditango_shape_t shape;
  int32_t  S;     /* rows per partition, ceil(N/P); set by ditango_states_init */
  void*    O;     /* fp32 or bf16 elements, per shape.state_dtype */
  float*   LSE;
  int32_t* tc;
} ditango_states_t;

/* Bytes the caller must allocate for the cache of `shape` (the per-pair
 * state cache of the attention-state section, Fig. 6: one (OUT, LSE) state
 * per head and (query partition, KV partition) pair): *o_bytes for O
 * = H*P*P*S*d*e (e = 4 for fp32 states, 2 for bf16) and *lse_bytes for
 * LSE = H*P*P*S*4 (either pointer may be
 * NULL).  Returns their sum, or 0 if the shape is invalid (message in
 * ditango_last_error()).  No allocation, no device call. */
size_t ditango_states_bytes(const ditango_shape_t* shape, size_t* o_bytes, size_t* lse_bytes);

/* Bind caller-owned buffers to `st` and mark every pair empty (tc[] = -1:
 * no state cached yet, so the first step must compute every pair, as the
 * anchor step of the anchor-steps section does).  O and LSE must be 16-byte
 * aligned device pointers of the sizes above; tc a host array of P*P int32.
 * Nothing is copied or allocated; the buffers stay the caller's.
 * Errors: DITANGO_EINVAL. */
int ditango_states_init(ditango_states_t* st, const ditango_shape_t* shape,
                        void* O, float* LSE, int32_t* tc);

/* Fresh partial attention for every pair with mask[q][k] = 1 (COMPUTE), on
 * every head: the attention state of query partition q against KV partition
 * k, OUT = softmax(scale * Q_q K_k^T) V_k and LSE = log sum exp of those
 * scaled scores (attention-state section, the state definition before
 * Eq. 4), written over the pair's slot, overwriting the stale state.  Pairs
 * with mask = 0 (REUSE) are not touched and no work is launched for them.
 * Computes with bf16 inputs, fp32 accumulation, fp32 softmax statistics;
 * probabilities are rounded to bf16 before the product with V; OUT is
 * normalised by the fp32 sum of the unrounded probabilities (d = 72: of the
 * rounded ones) and stored in the cache's format, LSE in fp32.  Checks
 * before launching anything that every REUSE pair holds a state (tc >= 0),
 * else returns DITANGO_ENOCACHE.  Does not change tc (see
 * ditango_state_cache_update).  Errors: EINVAL, ENOCACHE, EHIP. */
int ditango_attn_partial(const void* Q, const void* K, const void* V,
                         const uint8_t* mask, ditango_states_t* st, void* stream);

/* Commit step `step` to the cache metadata (host only, no device work):
 * tc[p] = step for every pair with mask = 1; REUSE pairs keep their tc.
 * If reused_out is not NULL it receives uint8 [P][P] with 1 exactly where
 * the pair is reused this step.  A mask of all ones is an anchor step: every
 * t_c becomes `step` (anchor-step section).  Errors: EINVAL (step < 0, step
 * below an existing tc, or a REUSE pair that was never computed). */
int ditango_state_cache_update(ditango_states_t* st, const uint8_t* mask, int32_t step,
                               uint8_t* reused_out);

/* Compose (Eq. 4) the P pair states of every row into the final output:
 *   O   device fp32 [H][N][d],  LSE device fp32 [H][N] (natural log).
 * Reads every slot of the cache; every pair must hold a state (tc >= 0),
 * else DITANGO_ENOCACHE.  Errors: EINVAL, ENOCACHE, EHIP. */
int ditango_state_merge(const ditango_states_t* st, float* O, float* LSE, void* stream);

/* The partial attention of the COMPUTE pairs and the composition (Eq. 4)
 * of every row in one launch: what ditango_attn_partial followed by
 * ditango_state_merge computes (the same fresh states, stored into the same
 * slots; O and LSE [H][N][d], [H][N] as ditango_state_merge writes them, up
 * to the rounding of the composition's sums), without t_c changes.  One
 * block per (head, query partition, query-row tile) computes that row's
 * fresh pairs one after the other and then composes the rows' P states, so
 * the composition's memory traffic overlaps other blocks' matrix work
 * (DiTango page, ring-based composed attention: partial states are composed
 * as they are produced).  Every REUSE pair must hold a state (tc >= 0),
 * else DITANGO_ENOCACHE before any launch.  Errors: EINVAL, ENOCACHE, EHIP. */
int ditango_attn_partial_merge(const void* Q, const void* K, const void* V, const uint8_t* mask,
                               ditango_states_t* st, float* O, float* LSE, void* stream);

/* One denoising step of one layer (anchor steps included): the partial
 * attention of the COMPUTE pairs, the t_c update and the composition, i.e.
 * ditango_attn_partial, ditango_state_cache_update and ditango_state_merge
 * in that order, with every check done before anything is launched or any
 * t_c changes.  The device work is one ditango_attn_partial_merge launch on
 * `stream`.  reused_out as in ditango_state_cache_update (may be NULL).
 * Errors: EINVAL, ENOCACHE, EHIP. */
int ditango_step(const void* Q, const void* K, const void* V, const uint8_t* mask, int32_t step,
                 ditango_states_t* st, float* O, float* LSE, uint8_t* reused_out, void* stream);

/* Selection mask of denoising step `step` under one of the locality
 * policies the workloads use (DiTango page, state-selection section: COMPUTE
 * or REUSE per unit and step; the near partitions matter most, Fig. 5a;
 * anchor-step section: an anchor step computes every unit).  Writes uint8
 * [P][P] (row q = query partition, column k = KV partition, 1 = COMPUTE):
 *   step 0                every pair fresh whatever the policy (the anchor
 *                         step that fills the cache)
 *   step >= 1:
 *   DITANGO_MASK_ALL      every pair fresh
 *   DITANGO_MASK_NONE     every pair reused
 *   DITANGO_MASK_RADIUS   fresh iff |q - k| <= n
 *   DITANGO_MASK_NEAREST  per row q, the n partitions k with the smallest
 *                         |q - k|, ties to the lower k
 *   DITANGO_MASK_RANDOM   per row q, q plus n-1 distinct others drawn with
 *                         SplitMix64 seeded with seed + step: rows in order,
 *                         candidates c = [k != q] ascending, for i < n-1 swap
 *                         c[i] with c[i + next() % (P-1-i)], take c[0..n-2]
 * `seed` is the workload's seed base (a workload with id c uses 1000 c), so a
 * step's random mask depends on (workload, step) only.  The mask is owned by
 * the caller.  Errors: EINVAL (NULL mask_out, bad policy, P outside 1..32,
 * step < 0, or from step 1 on n outside its range for the policy). */
#define DITANGO_MASK_ALL     0
#define DITANGO_MASK_NONE    1
#define DITANGO_MASK_RADIUS  2
#define DITANGO_MASK_NEAREST 3
#define DITANGO_MASK_RANDOM  4
int ditango_mask_build(int32_t policy, int32_t P, int32_t n, uint64_t seed, int32_t step,
                       uint8_t* mask_out);

/* Window attention with residual sharing at partition granularity (the
 * DiTFastAttn page: window attention plus a cached full-minus-window
 * residual), on the per-pair states.  window [P][P] (host, 0/1, at least one
 * 1 per row) names the window partitions of every query partition.
 *   DITANGO_WR_FULL    every pair must hold a state: O, LSE = composition of
 *                      all P states (full attention when all are fresh), and
 *                      R = O - (composition of the window states)
 *   DITANGO_WR_WINDOW  the window pairs must hold states: O = composition of
 *                      the window states + R, LSE = that composition's LSE
 * R: device fp32 [H][N][d] (caller-owned; written in FULL mode, read in
 * WINDOW mode).  O, LSE as for ditango_state_merge.  Reads only the window
 * states in WINDOW mode.  Errors: EINVAL, ENOCACHE (a needed pair holds no
 * state), EHIP. */
#define DITANGO_WR_FULL   0
#define DITANGO_WR_WINDOW 1
int ditango_window_residual_merge(const ditango_states_t* st, const uint8_t* window, int32_t mode, float* R,
                                  float* O, float* LSE, void* stream);

/* ---------------------------------------------------------------------
 * Grouped, composed state cache (state-selection section: the p partition
 * states are grouped into groups of g adjacent partitions, the group that
 * holds the local state keeping g - 1; selective compute and reuse, Fig. 6:
 * the remote states are composed and the composite is cached; ring-based
 * composed attention: a fresh group state is the composition of its
 * members' partial states; Dynamic Group State Compose: groups are merged k
 * at a time when memory runs short, and an anchor step returns to g).
 *
 * Groups are fixed and contiguous: G_j = {j g, ..., min((j+1) g, P) - 1},
 * j < m = ceil(P/g).  Query partition q owns 1 + m slots:
 *   slot 0      the local pair (q, q)
 *   slot 1 + j  the composed state of G_j without q (empty, and never read
 *               or written, when G_j = {q})
 * Per step a slot is COMPUTE when any of its members is marked fresh in the
 * pair mask [P][P] (the local slot follows mask[q][q]), else REUSE.  A fresh
 * group state is computed in one pass over the keys of all its members,
 * which is their composition (Eq. 4) up to rounding.  The row merge composes
 * the non-empty slots.  Slot buffers are separate so that slots released by
 * a group merge can be freed:
 *   O[s]   device [H][P][S][d], fp32 or bf16 (shape.state_dtype); row r of
 *          (h, q) = query row q*S + r
 *   LSE[s] device fp32 [H][P][S]
 *   tc     host int32 [P][DITANGO_MAX_SLOTS]; tc[q][s] = last step slot s of
 *          q was computed (-1: never); entries of empty slots stay -1.
 * 1 + ceil(P/g) must not exceed DITANGO_MAX_SLOTS (g = 1 needs P <= 31).
 * --------------------------------------------------------------------- */
#define DITANGO_MAX_SLOTS 32

typedef struct {
  ditango_shape_t shape;
  int32_t  S;                      /* ceil(N/P), set by ditango_gstates_init  */
  int32_t  g0;                     /* group size at init and after a reset    */
  int32_t  g;                      /* current group size, g0 * (merge factors) */
  void*    O[DITANGO_MAX_SLOTS];   /* slot buffers; NULL beyond the used slots */
  float*   LSE[DITANGO_MAX_SLOTS];
  int32_t* tc;
} ditango_gstates_t;

/* Slots per query partition for group size g: 1 + ceil(P/g), or 0 if P or g
 * is out of range or the count exceeds DITANGO_MAX_SLOTS. */
int32_t ditango_group_slots(int32_t P, int32_t g);

/* Device bytes of ONE slot buffer for `shape`: *o_bytes for O[s] and
 * *lse_bytes for LSE[s] (either may be NULL).  Returns their sum, 0 if the
 * shape is invalid. */
size_t ditango_gstates_slot_bytes(const ditango_shape_t* shape, size_t* o_bytes, size_t* lse_bytes);

/* Bind ditango_group_slots(P, g) caller-owned slot buffers (16-byte aligned,
 * sizes above) and a host tc array of P * DITANGO_MAX_SLOTS int32; marks
 * every slot empty (tc = -1).  Errors: EINVAL. */
int ditango_gstates_init(ditango_gstates_t* st, const ditango_shape_t* shape, int32_t g,
                         void* const* O, float* const* LSE, int32_t* tc);

/* Fresh partial attention for every COMPUTE slot (see above) on every head,
 * written over the slot.  REUSE slots are not touched and get no work.
 * Checks first that every non-empty REUSE slot holds a state, else
 * DITANGO_ENOCACHE.  Does not change tc.  Errors: EINVAL, ENOCACHE, EHIP. */
int ditango_group_attn_partial(const void* Q, const void* K, const void* V, const uint8_t* mask,
                               ditango_gstates_t* st, void* stream);

/* The fresh states of every COMPUTE slot and the composition (Eq. 4) of the
 * non-empty slots of every row, in one launch: what
 * ditango_group_attn_partial followed by ditango_group_merge computes (the
 * same slot states; O and LSE equal up to the rounding order of the
 * composition), without tc changes.  One block per (head, query partition,
 * query-row tile) computes that row's COMPUTE slots one after the other and
 * then composes its rows (ring-based composed attention of the DiTango page:
 * states are composed as they are produced).  Every non-empty REUSE slot
 * must hold a state, else DITANGO_ENOCACHE before any launch.  O and LSE as
 * in ditango_group_merge.  Errors: EINVAL, ENOCACHE, EHIP. */
int ditango_group_attn_partial_merge(const void* Q, const void* K, const void* V, const uint8_t* mask,
                                     ditango_gstates_t* st, float* O, float* LSE, void* stream);

/* Commit step `step` (host only): tc[q][s] = step for every COMPUTE slot.
 * If computed_out is not NULL it receives uint8 [P][ditango_group_slots(P, g)]
 * with 1 exactly at the COMPUTE slots (empty slots 0).  Errors: EINVAL (step
 * < 0, below an existing tc, or a REUSE slot that was never computed). */
int ditango_group_cache_update(ditango_gstates_t* st, const uint8_t* mask, int32_t step,
                               uint8_t* computed_out);

/* Compose (Eq. 4) the non-empty slots of every row into O device fp32
 * [H][N][d] and LSE device fp32 [H][N].  Every non-empty slot must hold a
 * state, else DITANGO_ENOCACHE.  Errors: EINVAL, ENOCACHE, EHIP. */
int ditango_group_merge(const ditango_gstates_t* st, float* O, float* LSE, void* stream);

/* Dynamic Group State Compose: group size g -> k*g, in place.  New group i
 * covers old groups k*i .. k*i+k-1; its state is their composition (Eq. 4,
 * empty ones skipped) written over old slot 1 + i, and its tc is the oldest
 * of theirs.  Slots >= ditango_group_slots(P, k*g) are released: their
 * pointers in `st` become NULL and the caller may free those buffers once
 * the stream has passed this call.  Every non-empty slot must hold a state,
 * else DITANGO_ENOCACHE; k >= 2.  Errors: EINVAL, ENOCACHE (both before any
 * work), EHIP (a launch failed part-way: the slot contents are then
 * undefined and the caller should reset and recompute at an anchor step). */
int ditango_group_compose(ditango_gstates_t* st, int32_t k, void* stream);

/* The memory trigger of Dynamic Group State Compose (DiTango page, dynamic
 * group state compose: when the cache's memory nears its limit, groups are
 * merged, repeatedly if need be, until an anchor step restores g0).  The
 * cache's device memory is (live slot count) x ditango_gstates_slot_bytes;
 * while it exceeds budget_bytes, groups are merged k at a time, each merge
 * as ditango_group_compose (k >= 2), enqueued on `stream`.  *merges_out (may
 * be NULL) receives the number of merges done, 0 when the cache already
 * fits.  The released slot buffers are the caller's to free once the stream
 * has passed the call.  Errors: EINVAL before any merge (bad k, or even one
 * group of all P partitions -- 2 slots -- exceeds the budget), ENOCACHE
 * (a non-empty slot holds no state), EHIP as ditango_group_compose. */
int ditango_group_fit(ditango_gstates_t* st, size_t budget_bytes, int32_t k, void* stream, int32_t* merges_out);

/* Return to the original group size g0 before an anchor step: binds
 * ditango_group_slots(P, g0) slot buffers (kept ones may be passed again)
 * and marks every slot empty.  Errors: EINVAL. */
int ditango_group_reset(ditango_gstates_t* st, void* const* O, float* const* LSE);

/* Group-aligned locality mask (state-selection section: selection per group;
 * locality of Fig. 5a): writes the pair mask uint8 [P][P] with, per query
 * partition q, mask[q][q] = 1 and every member of the n groups nearest to q
 * set, where a group's distance is min |q - k| over its members k != q
 * (groups that are {q} alone are skipped) and ties go to the lower group
 * index.  Every group is then wholly COMPUTE or wholly REUSE.  Errors:
 * EINVAL (P outside 1..32, g < 1, n < 0). */
int ditango_group_mask_build(int32_t P, int32_t g, int32_t n, uint8_t* mask_out);

/* ---- Anchor-guided selection (planner) ----
 *
 * Error-analysis and state-selection sections (Eq. 5-9, Algorithm 1): the
 * Attention State Error of a cached state is its importance w (its
 * normalised composition weight) times an error that grows with its cache
 * age; per query partition the KV partitions are grouped (groups of g
 * adjacent partitions, the local one apart and always computed), a group is
 * computed when the sum of its members' ASE exceeds a threshold eps and
 * reused otherwise; anchor steps compute everything, are triggered when the
 * local state drifts too far, and re-measure w, the scale ratios alpha and
 * eps (a percentile of the errors corrected at the anchor, set by a target
 * reuse fraction).  The page's equations are lost in extraction; this
 * library's model:
 *   signature of a pair state: the mean of its OUT rows, per head (d values);
 *   drift(a, b) = ||a - b|| / ||b|| over the heads' signatures concatenated;
 *   D(q, t): drift of q's local signature at step t against the last anchor;
 *   anchor at step < warmup (>= 2) or when max_q D(q, t) > drift_max;
 *   at an anchor: w(q,k) = pair importance averaged over heads, e(q,k) =
 *   drift of the pair's signature against the one cached before the step,
 *   alpha(q,k) = e(q,k) / D(q,t) (0 if D = 0), E(q,G) = sum over members of
 *   w e, eps = the ceil(target_reuse * n)-th smallest of the n values E
 *   (-inf if that is 0); per-group records Dc(q,G) = 0;
 *   between anchors: ASE(q,G) = sum over members k of w(q,k) alpha(q,k)
 *   max(0, D(q,t) - Dc(q,G)); G is computed iff ASE > eps, and then
 *   Dc(q,G) = D(q,t).
 * In E and ASE a member of zero importance adds nothing (also when its drift
 * or alpha is +inf), and ASE is 0 while D(q,t) <= Dc(q,G).
 * Groups: G_j = {j g .. min((j+1) g, P) - 1} without q; empty ones skipped. */

/* Per-pair statistics of the cache after a step's merge, on `stream`:
 *   W   device fp32 [H][P][P]: W[h][q][k] = mean over q's rows r of
 *       exp(LSE_slot(h,q,k)[r] - LSE[h][q*S + r]) for every pair -- the
 *       share of q's attention mass on k's keys;
 *   SIG device fp32 [H][P][P][d], 16-byte aligned: for the pairs with
 *       select[q][k] = 1 (host uint8 [P][P]) the mean of the slot's OUT rows;
 *       other entries are not touched (SIG may be NULL if none is selected).
 * LSE is the merged device fp32 [H][N] of the same cache contents.  W may be
 * NULL (importance not wanted, LSE not read: only the selected pairs are
 * visited).  Every pair must hold a state.  Errors: EINVAL, ENOCACHE, EHIP. */
int ditango_pair_stats(const ditango_states_t* st, const float* LSE, const uint8_t* select, float* W, float* SIG,
                       void* stream);

/* Drift of pair signatures between two device tables A and B, fp32
 * [H][P][P][d]: for the pairs with select[q][k] = 1 (host uint8 [P][P]),
 * out[q*P + k] = ||A - B|| / ||B|| over the pair's H*d values (0 when both
 * are 0, +inf when only B is); out is device fp32 [P][P], other entries
 * untouched.  Errors: EINVAL (NULL A, B, out or select, H or d < 1, P
 * outside 1..32, H*d >= 2^31, a select entry other than 0 or 1), EHIP. */
int ditango_sig_drift(const float* A, const float* B, int32_t H, int32_t P, int32_t d, const uint8_t* select,
                      float* out, void* stream);

/* Planner state (host only; set by ditango_planner_init and kept by the
 * calls below).  It works on scalars: the drifts and importances are
 * reduced on the GPU (ditango_pair_stats, ditango_sig_drift). */
typedef struct {
  int32_t P, g, H, warmup;
  float   target_reuse;   /* share of groups to reuse at the anchor error level, 0..1 */
  float   drift_max;      /* anchor when a local state drifts more than this */
  int32_t anchor;         /* decision of the last ditango_planner_plan */
  int32_t n_anchors, last_anchor;
  double  eps;
  double  D[DITANGO_MAX_P];
  double  W[DITANGO_MAX_P][DITANGO_MAX_P];
  double  alpha[DITANGO_MAX_P][DITANGO_MAX_P];
  double  Dc[DITANGO_MAX_P][DITANGO_MAX_P];   /* [q][group] */
} ditango_planner_t;

/* Errors: EINVAL (P outside 1..32, g outside 1..P, H < 1, target_reuse
 * outside [0, 1], drift_max < 0, warmup < 2, NULL planner). */
int ditango_planner_init(ditango_planner_t* pl, int32_t P, int32_t g, int32_t H, float target_reuse,
                         float drift_max, int32_t warmup);

/* Mask for step `step` (host uint8 [P][P], 1 = compute) from drift, host
 * fp32 [P]: D(q, t), the drift of q's freshly computed local signature
 * against the one at the last anchor (compute the local pairs first; read
 * only after the first anchor, may be NULL before).  A NaN drift counts as
 * beyond any bound.  *anchor_out (may be NULL) = 1 for an anchor step (mask
 * all ones).  Errors: EINVAL. */
int ditango_planner_plan(ditango_planner_t* pl, int32_t step, const float* drift, uint8_t* mask_out,
                         int32_t* anchor_out);

/* After step `step` ran with `mask`.  At an anchor step (the last plan
 * returned one) it reads W, host fp32 [H][P][P], the importance of the cache
 * after the step (ditango_pair_stats), and e, host fp32 [P][P] (diagonal not
 * read), each pair's signature drift against the signature it had before the
 * step (ditango_sig_drift; NULL at the first anchor); between anchors it reads
 * only the mask (W and e may be NULL).  Errors: EINVAL (an uninitialised
 * planner, a bad mask, step < 0, W NULL at an anchor, a W entry that is not
 * finite and >= 0, an off-diagonal e entry that is NaN or < 0; e may hold
 * +inf); nothing is changed on an error. */
int ditango_planner_update(ditango_planner_t* pl, int32_t step, const uint8_t* mask, const float* W,
                           const float* e);

/* Message of the last failed call on this thread ("" if none). */
const char* ditango_last_error(void);

/* Library ABI version (this header: 3). */
int32_t ditango_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DITANGO_H */
