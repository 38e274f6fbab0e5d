/*
 * apmoe.h - C ABI of libapmoe, an MI355X (gfx950) MoE expert-FFN layer over
 * any-precision (bit-plane + LUT) expert weights.
 *
 * Method: each expert's weights are stored once as bit-planes plus per-row
 * lookup tables and can be served at 3, 4, 5 or 6 bits or in an fp16
 * fallback, switched at run time per expert ("内存的饥饿游戏：当 MoE 权重与
 * KV 缓存争夺 GPU 的每一字节", zhichai.net, section "核心洞察：权重也能分页").
 * A quality-aware planner picks the bitwidths under a memory budget (same
 * page, sections "三层感知" and "安全边界与异步搬运"; "动态量化优化MoE模型服务",
 * time-frame.cloud, section "方法与技术路线") and the new plan takes effect at
 * a safe boundary between layer calls.
 *
 * Conventions (every entry point):
 *  - Returns 0 (APMOE_OK) or a negative APMOE_E* code; apmoe_strerror names it.
 *    Arguments are validated on the host before anything is enqueued; on an
 *    error nothing is launched and no output is touched.
 *  - The layer entry points (apmoe_route, apmoe_route_stats, apmoe_permute,
 *    apmoe_bitplane_lut_gemm, apmoe_combine, apmoe_commit_bits,
 *    apmoe_pack_planes, apmoe_exp_decode) work on caller-owned buffers only:
 *    they never allocate, free or synchronise; all GPU work is enqueued on
 *    `stream` (a hipStream_t; NULL means the default stream) in call order.
 *    No global mutable state: calls on different streams may run concurrently
 *    if their buffers are disjoint.  The host-only calls (planners, arena,
 *    exponent encoder) touch no GPU.  The pager (apmoe_pager_*) is the one
 *    stateful object: its block below lists what it allocates and where it
 *    waits on the host.
 *  - Pointers are device pointers unless marked [host].  fp16 values travel
 *    as uint16_t bit patterns (IEEE binary16).
 *  - T = 0 is a successful no-op.
 *
 * Shapes: T tokens, E experts, H hidden, I expert intermediate, k top-k,
 * slots S = T*k, slot s = t*k + j.  H and I must be multiples of 32.
 */
#ifndef APMOE_H
#define APMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define APMOE_OK        0
#define APMOE_EINVAL   (-1)   /* bad shape, null required pointer, bad stage */
#define APMOE_EBITS    (-2)   /* a bitwidth outside {3,4,5,6,16} */
#define APMOE_ENOSPACE (-3)   /* workspace too small, or planner budget infeasible */
#define APMOE_EHIP     (-4)   /* the HIP runtime reported an error at launch */

#define APMOE_GATE_UP_SWIGLU 0
#define APMOE_DOWN           1
/* Optional flags or-ed into `stage`: launch only one of the two paths
 * (e.g. to run them on two streams, or to time them apart).  Neither flag
 * (the default) launches both. */
#define APMOE_ONLY_GEMV   0x10
#define APMOE_ONLY_TILE   0x20

#define APMOE_MAX_EXPERTS 256

/*
 * One weight matrix W [rows x cols], cols = the contraction dimension K.
 * Two layouts of the six uint32 bit-planes exist:
 *  - canonical (interchange): planes[p][row][w], plane 0 = most significant
 *    bit of each weight's 6-bit code, bit i of word w = column 32*w + i;
 *    a b-bit code is the top b planes.  This is what checkpoints, the
 *    generator and the CPU oracle use.
 *  - packed (what the kernels read, from apmoe_pack_planes): every plane is
 *    still its own slab, so a b-bit expert reads only planes 0..b-1, but
 *    inside a slab the words of each 16-row group are ordered
 *    [step][g][i] = canonical word 4*step + g of row 16*group + i, with
 *    nsteps = ceil(cols/128) steps (missing words zero).  One slab holds
 *    rows * 4 * nsteps words; one GPU load then reads 256 contiguous bytes.
 *  planes : packed uint32 planes (see apmoe_packed_plane_words).
 *  lut[b-3]: fp16 [rows][1 << b], the b-bit centroid table of every row.
 *  w16    : fp16 [rows][cols] plain weights, read only when the expert runs
 *           at bitwidth 16; may be NULL for experts that never do.
 * All pointers are device pointers; planes and lut may be NULL for an expert
 * that only ever runs at 16 bits.
 */
typedef struct apmoe_mat {
    const uint32_t* planes;
    const uint16_t* lut[4];
    const uint16_t* w16;
} apmoe_mat;

/* gate and up are [I x H]; down is [H x I]. */
typedef struct apmoe_expert {
    apmoe_mat gate, up, down;
} apmoe_expert;

/*
 * Router: the top-k softmax gate of the MoE layer whose experts the bitwidth
 * plan serves ("内存的饥饿游戏：当 MoE 权重与 KV 缓存争夺 GPU 的每一字节",
 * zhichai.net, section "三层感知：离线 + 路由 + 提示词": the router's choices are
 * what the planner watches; the pages give no formula, so the plain top-k
 * softmax is read):
 * logits[t][e] = scale * (sum_h x[t][h] * w_router[e][h] + bias[e]),
 * products and sums in float64; the top k experts by logit (ties to the lower
 * index), listed by descending logit; gates = softmax over the k chosen logits.
 *  x        fp16 [T][H]          w_router fp32 [E][H]
 *  bias     fp32 [E] or NULL     logit_scale > 0
 *  topk_ids int32 [T][k] (out)   topk_w   fp32 [T][k] (out)
 *  x_norms  fp32 [T] (out) or NULL: ||x_t||_2 (squares summed in fp32 in a
 *           fixed order), computed from the x rows the router already reads;
 *           apmoe_permute turns them into the planner's routing statistics.
 *  ws/ws_bytes  workspace of at least apmoe_workspace_bytes(T, k, E, H, I)
 *           bytes, 8-byte aligned.  A few tokens over a small router matrix,
 *           or a single 16-expert tile with an unsplit hidden dimension, need
 *           none; otherwise partial fp64 logits are staged there for a
 *           second launch that adds them and selects.  APMOE_ENOSPACE if
 *           the buffer is short.
 * x and w_router must be 16-byte aligned.  Needs 1 <= k <= E <=
 * APMOE_MAX_EXPERTS, H > 0, H % 32 == 0 and T * k <= 2^30.
 */
int apmoe_route(const uint16_t* x, int T, int H, const float* w_router, const float* bias,
                float logit_scale, int E, int k, int32_t* topk_ids, float* topk_w, float* x_norms,
                void* ws, size_t ws_bytes, void* stream);

/*
 * Routing statistics for the bitwidth planner, over the slots of one
 * apmoe_route call ("内存的饥饿游戏：当 MoE 权重与 KV 缓存争夺 GPU 的每一字节",
 * zhichai.net, section "三层感知：离线 + 路由 + 提示词": a live measure of how
 * much routing each expert receives protects the busy experts, and a
 * correction taken from routing-weighted input norms adjusts the offline
 * sensitivity table for the current prompt).
 *  mass[e]  = sum over slots (t, j) with topk_ids[t][j] == e of topk_w[t][j]
 *  wnorm[e] = the same sum of topk_w[t][j] * ||x_t||_2
 *  x fp16 [T][H]; topk_ids int32 [T][k] and topk_w fp32 [T][k] as apmoe_route
 *  wrote them; mass, wnorm fp32 [E] (out), fp32 sums in a fixed order.
 *  ws/ws_bytes  at least T * 4 bytes (the token norms); APMOE_ENOSPACE if short.
 * Needs 1 <= k <= E <= APMOE_MAX_EXPERTS, H > 0 and H % 32 == 0; T = 0 gives
 * zeros.
 */
int apmoe_route_stats(const uint16_t* x, int T, int H, const int32_t* topk_ids, const float* topk_w, int k,
                      int E, float* mass, float* wnorm, void* ws, size_t ws_bytes, void* stream);

/*
 * Group slots by expert, so that each expert streams its bit-planes once for
 * all the tokens routed to it (the per-expert bitwidth of "内存的饥饿游戏：当 MoE
 * 权重与 KV 缓存争夺 GPU 的每一字节", zhichai.net, section "核心洞察：权重也能分页"
 * is a property of the expert, so its tokens are processed together): a
 * histogram, a scan and a stable permute (within an expert, slots in
 * ascending order).
 * Each token owns kk = k + n_shared slots.  n_shared >= 0 always-on experts
 * (a shared expert split into n_shared experts of the routed size, each taking
 * every token with weight 1) come first: slot t*kk + j is expert j for
 * j < n_shared and expert n_shared + topk_ids[t][j - n_shared] otherwise, so
 * the grouping covers E2 = E + n_shared experts and S = T*kk slots.
 *  counts[e]       number of slots of expert e                    int32 [E2]
 *  offsets[e]      exclusive prefix sum of counts, offsets[E2] = S int32 [E2+1]
 *  sorted_slots[p] slot at sorted position p                      int32 [S]
 *  pos_of_slot[s]  sorted position of slot s (inverse)            int32 [S]
 * Every topk_ids entry must lie in [0, E); E2 <= APMOE_MAX_EXPERTS.
 * Routing statistics in the same launch (optional; the same sums as
 * apmoe_route_stats, for the E routed experts): with mass != NULL, also
 *  mass[e]  = sum of topk_w over the slots routed to e              fp32 [E]
 *  wnorm[e] = sum of topk_w * x_norms[t] over the same slots        fp32 [E]
 * summed in a fixed order from topk_w fp32 [T][k] and x_norms fp32 [T] (as
 * apmoe_route wrote them); ws/ws_bytes must then hold S * 8 bytes
 * (APMOE_ENOSPACE otherwise).  With mass == NULL, topk_w, x_norms, wnorm and
 * ws are ignored (pass NULL, 0).
 */
int apmoe_permute(const int32_t* topk_ids, int T, int k, int E, int n_shared, int32_t* counts,
                  int32_t* offsets, int32_t* sorted_slots, int32_t* pos_of_slot, const float* topk_w,
                  const float* x_norms, float* mass, float* wnorm, void* ws, size_t ws_bytes, void* stream);

/*
 * One stage of every routed expert's FFN over its group of slots, reading each
 * expert's weights at that expert's own bitwidth: the top b bit-planes plus
 * the b-bit per-row lookup table, or the fp16 fallback
 * ("内存的饥饿游戏：当 MoE 权重与 KV 缓存争夺 GPU 的每一字节", zhichai.net, section
 * "核心洞察：权重也能分页": one stored weight set serves 3, 4, 5 or 6 bits, nested
 * by bit-plane, with 16 bits as the fallback).
 *  stage APMOE_GATE_UP_SWIGLU (optionally | APMOE_ONLY_GEMV or | APMOE_ONLY_TILE):
 *        in = x fp16 [T][H]; the row for sorted position
 *        p is x[sorted_slots[p] / k]; out = A fp16 [S][I] in sorted order,
 *        A = silu(W_gate x) * (W_up x), with g, u and silu in fp32.
 *  stage APMOE_DOWN: in = A fp16 [S][I] (sorted order); out = Y fp32 [S][H]
 *        in sorted order, Y = W_down a.
 *  experts  device array of E descriptors
 *  bits     int8 [E] on the device, each in {3,4,5,6,16}, read by the kernels
 *           (see apmoe_commit_bits); experts with no slots read no weights.
 *  offsets  int32 [E+1] from apmoe_permute; sorted_slots int32 [S].
 *  mfma_min_tokens  groups with at least this many slots take the dequantise-
 *           to-LDS + MFMA tile path, smaller ones the bit-plane GEMV path
 *           (both paths give results within the same tolerance).  >= 1.
 *           A token holds at most one slot of each expert, so when
 *           T < mfma_min_tokens every group takes the GEMV path and no tile
 *           kernel is launched.
 *  ws/ws_bytes  workspace of at least apmoe_workspace_bytes(T, k, E, H, I)
 *           bytes (split-K partial sums; 0 for shapes that never split K).
 *           Calls that share one workspace must not overlap.
 * The dispatch reads counts and bitwidths on the device: no host sync.
 * Limits: the kernels address `in` and every weight matrix with 32-bit byte
 * offsets, so T * H * 2 (gate/up) or T * k * I * 2 (down) bytes of input and
 * H * I * 2 bytes per matrix must each stay below 2 GiB (APMOE_EINVAL
 * otherwise); T * k <= 2^30.
 * An always-on shared expert whose intermediate size is n times I runs in the
 * same call as n extra fp16 experts (its gate/up row blocks and its down
 * column blocks) grouped by apmoe_permute with n_shared = n (pass E + n and
 * k + n here); any shared expert can also run alone as this call with E = 1,
 * bits = {16}, offsets = {0, T}, sorted_slots = 0..T-1 and k = 1.
 */
int apmoe_bitplane_lut_gemm(int stage, const apmoe_expert* experts, const int8_t* bits, int E,
                            const int32_t* offsets, const int32_t* sorted_slots, int k,
                            const uint16_t* in, void* out, int T, int H, int I,
                            int mfma_min_tokens, void* ws, size_t ws_bytes, void* stream);

/*
 * apmoe_bitplane_lut_gemm for callers that cannot allocate: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments and results as apmoe_bitplane_lut_gemm, without a workspace: the
 * split-K partial sums live in a static device array of
 * APMOE_NOALLOC_SCRATCH_BYTES inside the library (one per GPU, held until the
 * process ends; its address is looked up once per device on the first call).
 * The call allocates nothing.  It returns APMOE_ENOSPACE when the stage needs
 * more scratch than that (apmoe_workspace_bytes bounds the need; every shape
 * whose K is not split needs none) and APMOE_EHIP if the scratch address
 * cannot be looked up.  All calls on one GPU share its array: calls that
 * overlap on one GPU (on different streams) race; calls ordered on one
 * stream do not.
 */
#define APMOE_NOALLOC_SCRATCH_BYTES (16u << 20)
int apmoe_bitplane_lut_gemm_noalloc(int stage, const apmoe_expert* experts, const int8_t* bits, int E,
                                    const int32_t* offsets, const int32_t* sorted_slots, int k,
                                    const uint16_t* in, void* out, int T, int H, int I,
                                    int mfma_min_tokens, void* stream);

/*
 * Weighted combine of the experts' outputs into the layer output, the last
 * step of the MoE layer whose experts run at mixed bitwidths ("内存的饥饿游戏：
 * 当 MoE 权重与 KV 缓存争夺 GPU 的每一字节", zhichai.net, section "核心洞察：权重也能
 * 分页"; the pages give no formula, the plain gate-weighted sum is read), in a
 * fixed order with no atomics, kk = k + n_shared slots per token (as
 * apmoe_permute):
 *   out[t][h] = sum_{j=0..k-1} topk_w[t][j] * Y[pos_of_slot[t*kk + n_shared + j]][h]
 *             + sum_{j=0..n_shared-1} Y[pos_of_slot[t*kk + j]][h]  (+ y_shared[t][h]),
 * summed in fp32 in that order, rounded once to fp16.
 *  Y fp32 [T*kk][H] (sorted order); y_shared fp32 [T][H] or NULL; out fp16 [T][H].
 */
int apmoe_combine(const float* Y, const int32_t* pos_of_slot, const float* topk_w, int T, int k,
                  int n_shared, int H, const float* y_shared, uint16_t* out, void* stream);

/*
 * Greedy bitwidth planner (host only, touches no GPU).  Starting from every
 * expert at levels[0], it repeatedly lowers by one level the expert, not yet
 * at its floor, whose step costs the least harm per byte saved,
 * (harm[e][l+1] - harm[e][l]) / (bytes[e][l] - bytes[e][l+1]), ties to the
 * larger saving and then the lower index, until the plan fits the budget.
 *  levels    [host] int8 [L] bitwidths from high to low, e.g. {16,6,5,4,3}
 *  harm      [host] double [E][L]   bytes [host] uint64 [E][L] strictly decreasing in l
 *  floor_bits[host] int8 [E], each one of levels
 *  bits_out  [host] int8 [E]
 * Returns APMOE_ENOSPACE with bits_out = the floors when even the floors do
 * not fit; APMOE_EINVAL / APMOE_EBITS for malformed inputs.
 */
int apmoe_plan_bitwidths(int E, int L, const int8_t* levels, const double* harm,
                         const uint64_t* bytes, const int8_t* floor_bits, uint64_t budget,
                         int8_t* bits_out);

/*
 * Planner inputs from routing statistics (host only).  The offline harm table
 * is corrected per expert by what apmoe_route_stats measured
 * ("内存的饥饿游戏：当 MoE 权重与 KV 缓存争夺 GPU 的每一字节", zhichai.net, section
 * "三层感知：离线 + 路由 + 提示词": busy experts are protected, and a residual from
 * routing-weighted input norms adjusts the offline sensitivity to the current
 * prompt; no formula is given, the plain reading is):
 *   load[e]  = mass[e] / mean over experts of mass
 *   resid[e] = (wnorm[e] / mass[e]) / (sum of wnorm / sum of mass), 1 if mass[e] = 0
 *   mult[e]  = load[e] * resid[e]            (1 everywhere if nothing was routed)
 * in double precision, sums in index order.
 *  mass, wnorm [host] fp32 [E] (>= 0, as apmoe_route_stats wrote them);
 *  mult [host] double [E] (out).  APMOE_EINVAL for a negative or NaN input.
 * apmoe_plan_routed runs apmoe_plan_bitwidths on harm[e][l] * mult[e] (same
 * arguments and returns, plus mass and wnorm).
 */
int apmoe_harm_multipliers(int E, const float* mass, const float* wnorm, double* mult);
int apmoe_plan_routed(int E, int L, const int8_t* levels, const double* harm, const uint64_t* bytes,
                      const int8_t* floor_bits, uint64_t budget, const float* mass, const float* wnorm,
                      int8_t* bits_out);

/*
 * Commit a plan at a safe boundary ("内存的饥饿游戏：当 MoE 权重与 KV 缓存争夺 GPU
 * 的每一字节", zhichai.net, section "安全边界与异步搬运": a new bitwidth plan takes
 * effect only between layer calls): validates bits_host [host] int8 [E] and
 * enqueues its copy into bits_dev on `stream`, so layer calls enqueued before
 * it see the old bitwidths and calls enqueued after it see the new ones.  The
 * values travel as kernel arguments: bits_host may be reused on return.
 */
int apmoe_commit_bits(const int8_t* bits_host, int E, int8_t* bits_dev, void* stream);

/*
 * One step of the online bitwidth planner as the KV cache grows or shrinks
 * (host only).  The weight budget is M_w = max(0, m_total - m_kv)
 * ("动态量化优化MoE模型服务", time-frame.cloud, section "方法与技术路线"); the
 * search walks bitwidth stages from the safest to the most aggressive and
 * stops at the first that fits, never below an expert's floor ("内存的饥饿游戏：
 * 当 MoE 权重与 KV 缓存争夺 GPU 的每一字节", zhichai.net, section "安全边界与异步搬运").
 *  levels, harm, bytes, floor_bits  as apmoe_plan_bitwidths (host arrays)
 *  stage_bits [n_stages]  lowest bitwidth of each stage, safest first (each one
 *                         of levels); in stage s an expert's floor is the
 *                         higher of floor_bits[e] and stage_bits[s]
 *  hysteresis             the current plan is kept while it fits M_w with less
 *                         than this many bytes to spare; otherwise the plan is
 *                         recomputed for M_w - hysteresis, then for M_w
 *  bits_now [E]           the current plan;  bits_out [E] the new plan
 *  stage_out              stage of the new plan, -1 when the current plan is kept
 * Returns APMOE_OK, or APMOE_ENOSPACE with every expert at its last-stage
 * floor when no stage fits; APMOE_EINVAL / APMOE_EBITS on bad input.
 */
int apmoe_plan_online(int E, int L, const int8_t* levels, const double* harm, const uint64_t* bytes,
                      const int8_t* floor_bits, int n_stages, const int8_t* stage_bits, uint64_t m_total,
                      uint64_t m_kv, uint64_t hysteresis, const int8_t* bits_now, int8_t* bits_out,
                      int* stage_out);

/* Workspace bytes apmoe_route (over up to E experts) and
 * apmoe_bitplane_lut_gemm need for these shapes (one buffer serves both;
 * calls that share it must not overlap). */
size_t apmoe_workspace_bytes(int T, int k, int E, int H, int I);

/* uint32 words of all six packed planes of a rows x cols matrix:
 * 6 * rows * 4 * ceil(cols / 128). */
size_t apmoe_packed_plane_words(int rows, int cols);

/*
 * Reorder canonical planes [6][rows][cols/32] into the packed layout the
 * kernels read (a one-time weight preparation, not part of a layer call).
 *  src  device, canonical planes;  dst  device, apmoe_packed_plane_words()
 *  words, must not overlap src.  rows % 16 == 0 and cols % 32 == 0.
 */
int apmoe_pack_planes(const uint32_t* src, int rows, int cols, uint32_t* dst, void* stream);

/* Static description of an error code. */
const char* apmoe_strerror(int code);

/*
 * Plane paging ("内存的饥饿游戏：当 MoE 权重与 KV 缓存争夺 GPU 的每一字节",
 * zhichai.net, sections "核心洞察：权重也能分页" and "安全边界与异步搬运": the
 * bit-planes are the pages, moved between GPU and host asynchronously and
 * committed at a safe boundary so that the movement hides behind inference).
 *
 * apmoe_arena_*: a host-side first-fit allocator over an address range
 * [0, bytes) in 256-byte units; it never touches memory, so it runs without a
 * GPU.  Free ranges are kept coalesced.
 *  create   bytes rounded down to 256; *out owned by the caller (destroy).
 *  alloc    first free range (lowest offset) that holds bytes (rounded up to
 *           256); APMOE_ENOSPACE if none.
 *  take     claim exactly [off, off + bytes) if all of it is free, else
 *           APMOE_ENOSPACE; off must be 256-aligned.
 *  release  return [off, off + bytes); APMOE_EINVAL (and no change) if any
 *           of it lies outside the range or is already free.
 *  stats    free bytes, largest free range, number of free ranges (any may be NULL).
 */
typedef struct apmoe_arena apmoe_arena;
int apmoe_arena_create(uint64_t bytes, apmoe_arena** out);
void apmoe_arena_destroy(apmoe_arena* arena);
int apmoe_arena_alloc(apmoe_arena* arena, uint64_t bytes, uint64_t* off);
int apmoe_arena_take(apmoe_arena* arena, uint64_t off, uint64_t bytes);
int apmoe_arena_release(apmoe_arena* arena, uint64_t off, uint64_t bytes);
int apmoe_arena_stats(const apmoe_arena* arena, uint64_t* free_bytes, uint64_t* largest, int* n_ranges);

/*
 * apmoe_pager_*: residency of E experts' bit-planes and LUTs in a device
 * arena.  An expert at b in {3..6} bits holds planes 0..b-1 of each of its
 * three matrices (one block per matrix, planes at the packed slab stride, so
 * the GEMM's addressing is unchanged) and the b-bit LUT of each; at 16 bits
 * it holds neither (its fp16 weights, which the caller places in the
 * descriptors, are not paged).
 *  create  host_planes [3E]: per expert gate, up, down, the six packed slabs
 *          (apmoe_packed_plane_words(rows, cols) words, as apmoe_pack_planes
 *          writes them); host_luts [3E][4]: fp16 [rows][1 << b] for b = 3..6.
 *          Read only during create: the pager keeps its own pinned copy
 *          (hipHostMalloc), laid out by promotion step and then expert, so
 *          that raising an expert by one bit is one contiguous range (and
 *          raising experts with adjacent indices to the same bitwidth too).
 *          arena: device memory (256-byte aligned, arena_bytes) owned by the
 *          caller; the pager keeps a patch buffer and a copy list (28 bytes
 *          x 18E) in it.  experts: the device
 *          descriptors of these E experts (gate/up/down planes and lut words
 *          are written by commits; w16 words are left alone); bits: their
 *          device bits table.  Nothing is resident until the first commit.
 *          APMOE_ENOSPACE if the arena cannot hold the patch buffer and copy
 *          list.
 *  stage   bits_new [E] (host): enqueue on copy_stream the copies that make
 *          the new residency and record what the commit retires.  The new
 *          planes and LUTs go host to device (one hipMemcpyAsync per expert
 *          and bitwidth step, on the copy engines) into a staging block of
 *          the arena, which the commit places; a block that cannot grow in
 *          place is moved, its resident planes copied device to device by the
 *          commit.  When the arena has no room for the staging block, each
 *          matrix's planes of one step and each LUT are copied host to device
 *          straight into place.  The staging block returns to the arena with
 *          the blocks the commit retires.  copy_stream gets copies only, no
 *          kernel or event (an event queued behind the copies would hold up,
 *          until they finish, every stream sharing its hardware queue); it
 *          must stay valid until the commit (or destroy).  The layer keeps
 *          running at the old bitwidths meanwhile.
 *          APMOE_EBITS for a bitwidth outside {3,4,5,6,16};
 *          APMOE_ENOSPACE (nothing staged, nothing enqueued) when the arena
 *          cannot hold the new blocks even after waiting for retired blocks;
 *          APMOE_EINVAL if a staged change is not yet committed (or, with
 *          nothing enqueued, if a planned copy fell outside the arena or the
 *          host copy).  Waits on the host for the previous commit to have
 *          executed.
 *  commit  on stream: record an event on the stage's copy_stream and wait for
 *          it (the staged copies), place the staged planes and LUTs and move
 *          the relocated blocks (one kernel, when there is anything to place),
 *          then write the plane and LUT pointers of every paged matrix and the
 *          bits table together (one kernel), so every later kernel on stream
 *          sees the new bitwidths and every earlier one the old.  Blocks the
 *          change retires return to the arena once the stream has passed the
 *          commit.  All kernels that read these experts must be ordered on
 *          stream.
 *  stats   resident plane and LUT bytes, arena free bytes and largest free
 *          range, the plane and LUT bytes the last stage copied host to
 *          device, the resident plane bytes it moved to new blocks, and the
 *          number of host-to-device ranges it copied (any pointer may be
 *          NULL).
 *  destroy waits for outstanding copies and commits; the arena stays the
 *          caller's.
 * Host resources and waits (the pager is the library's one stateful object):
 * create allocates the pager, its pinned host copy of the planes and LUTs
 * (as many bytes as all planes and LUTs of the E experts), a pinned patch
 * buffer and copy list (hipHostMalloc) and two HIP events, all freed by
 * destroy; a commit that retires blocks creates one more event, destroyed
 * once those blocks are back in the arena.  stage waits on the host
 * (hipEventSynchronize) for the previous commit to have run, and, when the
 * arena is short, for the retired blocks; if enqueueing a copy fails it
 * synchronises copy_stream before undoing the claims.  destroy synchronises
 * the copy_stream of a stage not yet committed and waits for the last
 * commit.
 * Needs 1 <= E <= APMOE_MAX_EXPERTS, H % 32 == 0, I % 32 == 0.
 */
typedef struct apmoe_pager apmoe_pager;
int apmoe_pager_create(int E, int H, int I, const void* const* host_planes, const void* const* host_luts,
                       void* arena, uint64_t arena_bytes, apmoe_expert* experts, int8_t* bits,
                       apmoe_pager** out);
int apmoe_pager_stage(apmoe_pager* pager, const int8_t* bits_new, void* copy_stream);
int apmoe_pager_commit(apmoe_pager* pager, void* stream);
int apmoe_pager_stats(apmoe_pager* pager, uint64_t* resident_bytes, uint64_t* free_bytes,
                      uint64_t* largest_free, uint64_t* h2d_bytes, uint64_t* d2d_bytes, uint64_t* copy_ranges);
int apmoe_pager_destroy(apmoe_pager* pager);

/*
 * Lossless exponent codec for fp16 weights ("专家分页机制：7倍MoE推理吞吐背后的
 * 显存解耦革命", mubeitech.com, the passage on its third mechanism,
 * bandwidth-balanced storage tiering: the exponent bits of floating-point
 * weights are Huffman-coded offline and decoded in GPU memory, in parallel
 * with host transfers).  Format: a weight's high byte (sign, exponent, top two
 * mantissa bits) is coded with a canonical Huffman code (ties: key (count,
 * id), leaves id = symbol, merged nodes 256, 257, ... in creation order),
 * lengths limited to 12 bits by raising every non-zero count to at least
 * total >> (12 - r), r = 2, 3, ..., until the code fits; the low byte is kept
 * raw.  Weights go in groups of 9216: block l (0..63) of group g holds
 * weights g*9216 + 64j + l, j = 0..min(144, (n - g*9216)/64) - 1; the bit
 * stream is the blocks' codes in block order, most significant bit first in
 * 32-bit words, ended by two zero words.
 *  plan    [host] w: n fp16 bit patterns (n > 0, n % 64 == 0, 12 n < 2^32);
 *          lengths[256] (out): code length per high byte (0 = absent);
 *          nwords, nblocks (out): stream words and blocks (64 per group).
 *  encode  [host] with those lengths: words[nwords] (APMOE_ENOSPACE if
 *          short), block_off[nblocks] = bit offset of each block, lo[n] = low
 *          bytes, table[4096] = (length << 8) | symbol for every 12-bit
 *          prefix.  APMOE_EINVAL for a high byte without a code.
 *  decode  [device] words, block_off, lo, table as encode wrote them -> out
 *          fp16 [n], bit-exact.  The stream is read within nwords words
 *          whatever it holds.
 */
int apmoe_exp_plan(const uint16_t* w, uint64_t n, uint8_t* lengths, uint64_t* nwords, uint64_t* nblocks);
int apmoe_exp_encode(const uint16_t* w, uint64_t n, const uint8_t* lengths, uint32_t* words, uint64_t nwords,
                     uint32_t* block_off, uint8_t* lo, uint16_t* table);
int apmoe_exp_decode(const uint32_t* words, uint64_t nwords, const uint32_t* block_off, const uint8_t* lo,
                     const uint16_t* table, uint64_t n, uint16_t* out, void* stream);

/* Up to APMOE_EXP_MAX_BATCH coded matrices decoded by one launch (the same
 * passage: a layer's fp16 weights are decoded together once they are in GPU
 * memory).  Host arrays of count entries, each entry as apmoe_exp_decode's
 * arguments (device pointers, each matrix with its own table); every entry
 * is validated before anything is launched.  A small matrix alone gives the
 * GPU less than one decoding wave per SIMD, and each wave's time is one
 * block's chain of dependent lookups, so decoding a layer's matrices
 * together takes about as long as decoding one of them. */
#define APMOE_EXP_MAX_BATCH 16
int apmoe_exp_decode_batch(int count, const uint32_t* const* words, const uint64_t* nwords,
                           const uint32_t* const* block_off, const uint8_t* const* lo, const uint16_t* const* table,
                           const uint64_t* n, uint16_t* const* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* APMOE_H */
