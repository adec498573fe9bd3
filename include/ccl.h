/*
 * ccl.h -- C ABI of libccl: the reduce and copy data plane of a collective
 * library, run on one GPU over P simulated rank buffers resident in its HBM.
 *
 * Sources (web pages this library is built from):
 *   [digest]  "NCCL M2N vs T-CCL" digest, lqnn.cn news 207677.
 *   [roadmap] "nccl-extensions" page, an explainer of NCCL's roadmap; its
 *             "NCCL API overview" table (host API collectives such as
 *             all-reduce) and its GENK section (ring all-gather,
 *             reduce-scatter, all-reduce built from receive/reduce/send parts).
 *
 * Conventions shared by every call:
 *   - Buffers are device memory (or memory the current device can address),
 *     owned by the caller.  The library never allocates or frees them.
 *     Pointer arrays (send[], recv[], src_bufs[], dst_bufs[]) are host arrays
 *     read only during the call.
 *   - Every pointer must be aligned to its element size.  16-byte aligned
 *     buffers take the wide vector path; anything else is still correct but
 *     runs a slower element-wise kernel.
 *   - stream is a hipStream_t (NULL = the null stream).  Work is enqueued on
 *     it and the call returns without waiting.  The library creates no
 *     streams and never synchronizes them.
 *   - Fail-stop: every argument is checked before anything is enqueued, so a
 *     return other than CCL_OK means no kernel was launched and no output byte
 *     was touched.  CCL_ERR_HIP reports a failed launch; faults inside a
 *     kernel surface at the caller's next synchronization.
 *   - A count of 0 is a valid no-op (pointers are then not inspected).
 *   - Host threads: any call may run concurrently with others from other
 *     threads, on the same or different streams.  Calls in flight together
 *     must not write a buffer another of them reads or writes; the stream
 *     order is the caller's to arrange.  A plan may be shared by concurrent
 *     calls (its device table is built once per device and chunk size under
 *     a lock); destroying it while another call still uses it is an error the
 *     library does not detect.
 *   - Reductions are computed per element as a fold in rank order 0..P-1 that
 *     starts from rank 0's value and accumulates in fp32 (bf16 and fp16
 *     inputs are widened exactly, the fp32 result is rounded back once, to
 *     nearest even; int32 sums wrap).  min and max keep the earlier rank's value on a
 *     tie.  Results therefore do not depend on the launch configuration.
 *     [digest] s2.1 gives the op set (add, min, max); the order and
 *     accumulator type are this library's choice, fixed so results are
 *     reproducible.
 */
#ifndef CCL_H
#define CCL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CCL_OK = 0,
    CCL_ERR_INVALID_ARG = 1, /* NULL pointer, bad count/P/dtype/op, misaligned pointer */
    CCL_ERR_UNSUPPORTED = 2, /* a valid request the library does not implement */
    CCL_ERR_ALIASING = 3,    /* buffers overlap in a way the op cannot run in place */
    CCL_ERR_LAYOUT = 4,      /* reshard layout violates a constraint */
    CCL_ERR_HIP = 5,         /* a HIP runtime call failed */
    CCL_ERR_NOMEM = 6,       /* host or device allocation for library state failed */
    CCL_ERR_SCRATCH_LIMIT = 7 /* the no-allocation entry point would need more than
                                 CCL_NOALLOC_SCRATCH_BYTES of scratch */
} ccl_status_t;

typedef enum { CCL_FLOAT32 = 0, CCL_BFLOAT16 = 1, CCL_INT32 = 2, CCL_FLOAT16 = 3 } ccl_dtype_t;

/* [digest] s2.1: the reduction operations the bulk-reduce primitive offers. */
typedef enum { CCL_SUM = 0, CCL_MIN = 1, CCL_MAX = 2 } ccl_op_t;

#define CCL_MAX_RANKS 16        /* P limit of the collectives */
#define CCL_MAX_MESH_DIMS 4     /* axes of a reshard mesh */
#define CCL_MAX_TENSOR_DIMS 8   /* dims of a resharded tensor */
#define CCL_MAX_MESH_RANKS 64   /* ranks of one reshard mesh */
#define CCL_NOALLOC_SCRATCH_BYTES (2u << 20) /* fixed scratch of the no-allocation entry point */

/*
 * Optional launch configuration ([digest] s2.3: the bulk-copy engine's launch
 * configuration is tuned by a sweep).  Pass NULL for the built-in defaults,
 * which come from such sweeps on MI355X (2 GiB of bf16 input over P ranks,
 * unless a rule names sizes; `python bench.py --defaults` and `--sweep`
 * re-measure every rule below against its alternatives):
 *   all-reduce      P = 1: 8 KiB chunks, unroll 1, <= 8 WGs per CU;
 *                   P = 2: 8 KiB chunks, unroll 2 (unroll 1 above 128 and
 *                   up to 256 MiB per rank), <= 8 WGs per CU; with
 *                   write-through stores 4 KiB chunks, unroll 1, <= 6 WGs
 *                   per CU;
 *                   P = 3, 4: 4 KiB chunks, unroll 1, <= 6 WGs per CU (with
 *                   write-through stores: 8 KiB chunks, <= 3 WGs per CU, but
 *                   4 KiB chunks at P = 4 from 512 MiB per rank when the
 *                   inputs do not all start at one offset modulo 2 MiB);
 *                   P >= 5: 4 KiB chunks, unroll 1, <= 3 WGs per CU; but
 *                   3 <= P <= 8 with 1-128 MiB per rank: 8 KiB chunks,
 *                   unroll 2, <= 4 WGs per CU; and from 512 MiB per rank
 *                   when every input starts at the same offset modulo 2 MiB
 *                   (separate framework allocations): 16 KiB chunks, <= 3
 *                   WGs per CU at 6 <= P <= 16, 8 KiB chunks, <= 3 WGs per
 *                   CU at P = 5
 *   reduce-scatter and reduce  register-direct, 8 KiB chunks, unroll 2,
 *                   <= 4 (P <= 2) or 3 WGs per CU, but 4 KiB chunks, unroll 1,
 *                   <= 4 WGs per CU for 9 <= P <= 12
 *   broadcast       as all-gather
 *   all-gather      P <= 3: register-direct, 8 KiB chunks, unroll 2, <= 4
 *                   (P <= 2) or 3 WGs per CU; 4 <= P <= 8: register-direct,
 *                   4 KiB chunks, unroll 1, <= 4 WGs per CU; P >= 9:
 *                   register-direct, 4 KiB chunks, unroll 1, <= 3 WGs per CU
 *                   (<= 4 with write-through stores)
 *   reshard copy    unroll 4; one replica per destination shard: 16 KiB
 *                   chunks, <= 4 WGs per CU, nontemporal loads and stores;
 *                   two or more: 32 KiB chunks, <= 2 WGs per CU,
 *                   nontemporal stores only (four or more: written through,
 *                   see store_policy)
 *   reshard + fp8   32 KiB chunks, unroll 2, no cap (the quantizing pass does
 *                   enough ALU work per byte that it needs every resident wave)
 *   all-reduce + RMSNorm  P >= 8 with rows of at least 8 KiB per rank:
 *                   the split-row form (chunk_bytes = 4096 below): a fold
 *                   pass with <= 4 WGs per CU and a norm pass with <= 2,
 *                   whose stores write through past 256 MiB per rank when
 *                   every output and row starts on 256 bytes.  Otherwise
 *                   one workgroup per row; <= 3 WGs per CU for rows of 4-8
 *                   KiB, otherwise residency bounded only by registers and
 *                   the row buffer it keeps in LDS; at P >= 6 rows longer
 *                   than 16 KiB take the row-pipelined kernel (stages = 2)
 *                   on a persistent grid of one workgroup per CU.  It reads
 *                   chunk_bytes (4096 or at least the row), workgroups,
 *                   stages (1 or 2; 3 and 4 give CCL_ERR_UNSUPPORTED),
 *                   nontemporal, occupancy (both passes of the split form)
 *                   and store_policy and ignores the rest
 * Buffers whose inputs sit at a different offset mod 16 from their outputs
 * use a register-direct kernel that realigns the inputs in VGPRs; unless the
 * caller sets them, it runs 4 KiB chunks with <= 8 WGs per CU (reduce-scatter
 * above P = 8: 8 KiB chunks, <= 4 WGs per CU; all-gather: <= 4 for P <= 6,
 * <= 3 above) and cacheable loads (nontemporal stores only; its all-reduce
 * and all-gather forms always load through the cache).
 * A zero field means "the default for this call"; out-of-range values give
 * CCL_ERR_INVALID_ARG.  None of these fields changes any result.
 *
 *   chunk_bytes  contiguous bytes of each rank buffer one workgroup owns per
 *                scheduling step (its share of a shard); a multiple of 16,
 *                at least 1024.  The LDS pipeline needs a multiple of its
 *                4096-byte tile: stages > 1 with another chunk size is
 *                rejected.
 *   workgroups   grid size; chunks are dealt to workgroups round-robin.
 *                Default: one workgroup per chunk.
 *   stages       1 = register-direct (loads land in VGPRs), 2..4 = LDS
 *                pipeline (never chosen by default: on MI355X it is level
 *                with the register-direct kernel on the all-reduce and
 *                behind it on the reduce-scatter and all-gather):
 *                producer waves stream tiles into a ring of
 *                `stages` LDS buffers with asynchronous global->LDS loads,
 *                consumer waves fold and store them (clamped so the ring
 *                fits in 128 KiB).  The reshard copy is register-direct only.
 *                For the fused RMSNorm: chunk_bytes = 4096 with rows longer
 *                than that selects the split-row form (one workgroup per
 *                4 KiB piece of a row in each of two passes); any other
 *                value below the row length gives CCL_ERR_UNSUPPORTED.
 *                For the fused RMSNorm: 1 = one row at a time per workgroup,
 *                2 = two rows software-pipelined (the next row's inputs are
 *                loaded and folded while the current row is stored).
 *   unroll       register-direct only: 16-byte vectors each lane keeps in
 *                flight per rank (1, 2 or 4; 4 is used as 2 when P > 8); for
 *                the fp8 reshard, vectors each lane loads before quantizing.
 *   nontemporal  bit 0: nontemporal loads, bit 1: nontemporal stores;
 *                0 = default (both; stores only for a reshard copy with
 *                replicated destinations), 4 = neither.  The register-direct
 *                collective kernel keeps one stream per call cacheable
 *                even so (one among P nontemporal streams measured 6-19 %
 *                faster than none): for the all-reduce the stores to the
 *                last rank's output (with write-through stores the loads
 *                of the first input instead; with unroll 2 the loads of
 *                the last rank's input as well), for the other
 *                collectives the loads of the first input.  The LDS
 *                pipeline does the same with write-through stores; with
 *                nontemporal ones it keeps output 0's stores cacheable for
 *                the all-reduce and all-gather and no stream for the
 *                reduce-scatter.
 *   occupancy    at most this many workgroups resident per compute unit
 *                (enforced by reserving LDS), 1..32; 32 is effectively no
 *                cap.  Fewer resident waves keep fewer DRAM pages open at
 *                once, which is what lets P-stream kernels reach the HBM
 *                bandwidth a single copy stream gets.
 *   store_policy how the nontemporal stores reach memory: 1 = write-through
 *                (the stores carry the device-scope bit as well, so the L2
 *                forwards each line to memory instead of keeping it dirty;
 *                collectives, reshard copy, FP8 reshard codes and fused
 *                RMSNorm, for chunks of up to 1 GiB), 2 = nontemporal only,
 *                0 = default:
 *                write-through for the all-reduce at P = 2 above 256 MiB
 *                per rank, at P = 3 from 256 MiB, at 4 <= P <= 8 above
 *                128 MiB and at 9 <= P <= 16 from 16 MiB, for
 *                reduce-scatter and reduce at P <= 8, for
 *                all-gather and broadcast at P = 2, at 7 <= P <= 16 with at
 *                most 256 MiB of input in all and at 4 <= P <= 6 with at most
 *                64 MiB (from P = 9 on with <= 4 WGs per CU instead of 3),
 *                for the reshard copy with four or more replicas per
 *                destination shard, each only where every
 *                output's stores start on a 256-byte boundary (partial lines
 *                written through cost far more than they save); nontemporal
 *                only for the other all-reduces, the other all-gathers and
 *                broadcasts, the other reshard copies, the FP8 reshard and
 *                the fused RMSNorm's one-pass forms (within +-1.3 % of
 *                write-through, either sign); the split-row RMSNorm as
 *                stated above.
 *                Write-through applies to the register-direct kernels and
 *                the LDS pipeline (not the realigning kernel); with it both
 *                keep input 0's loads cacheable.  It needs
 *                >= 4 resident workgroups per CU to cover its longer store
 *                completion in the all-gather; with fewer it can be much
 *                slower.  Ignored when nontemporal stores are off.
 */
typedef struct {
    uint64_t chunk_bytes;
    int32_t workgroups;
    int32_t stages;
    int32_t unroll;
    int32_t nontemporal;
    int32_t occupancy;
    int32_t store_policy;
} ccl_launch_config_t;

/*
 * All-reduce ([roadmap] API overview and GENK; [digest] s2.5, where an
 * all-reduce is a shard-in followed by a shard-out).  For every element index
 * i < count and every rank q: recv[q][i] = fold over r of send[r][i].
 * The two phases are fused: each shard's reduced value stays in registers and
 * is stored to all P outputs, so it never makes an extra trip through HBM.
 *
 *   send   P pointers, each to `count` elements of dtype.
 *   recv   P pointers, each to `count` elements of dtype.
 *   In place: recv[q] == send[q] is allowed (as is any recv[q] == send[r]);
 *   any other overlap between buffers, or of two recv buffers, gives
 *   CCL_ERR_ALIASING.
 */
ccl_status_t ccl_all_reduce(const void *const *send, void *const *recv, int nranks, size_t count,
                            int dtype, int op, void *stream, const ccl_launch_config_t *cfg);

/*
 * Reduce-scatter, the shard-in ([digest] s2.2: the owner of a shard loads
 * every peer's contribution and reduces it locally, with no cross-device
 * atomics; s2.3: the logical tensor is cut into P shards, shard s owned by
 * rank s).  For s < P, j < recvcount:
 *   recv[s][j] = fold over r of send[r][s*recvcount + j].
 *
 *   send   P pointers, each to P*recvcount elements.
 *   recv   P pointers, each to recvcount elements.
 *   In place: recv[s] == send[s] + s*recvcount elements is allowed (the
 *   NCCL convention); other overlaps give CCL_ERR_ALIASING.
 */
ccl_status_t ccl_reduce_scatter(const void *const *send, void *const *recv, int nranks,
                                size_t recvcount, int dtype, int op, void *stream,
                                const ccl_launch_config_t *cfg);

/*
 * All-gather, the shard-out ([digest] s2.2: the owner loads its final shard
 * once and stores that one copy to every peer).  For q, r < P, j < sendcount:
 *   recv[q][r*sendcount + j] = send[r][j].
 *
 *   send   P pointers, each to sendcount elements.
 *   recv   P pointers, each to P*sendcount elements.
 *   In place: send[r] == recv[r] + r*sendcount elements is allowed;
 *   other overlaps give CCL_ERR_ALIASING.  dtype only sets the element size.
 */
ccl_status_t ccl_all_gather(const void *const *send, void *const *recv, int nranks,
                            size_t sendcount, int dtype, void *stream,
                            const ccl_launch_config_t *cfg);

/*
 * All-reduce with RMSNorm fused between its two halves ([roadmap]: the Device
 * API example that fuses a Transformer RMSNorm with reduce-scatter and
 * all-gather in one kernel).  Every rank buffer is a rows x hidden row-major
 * matrix.  Per row t:
 *   s[h]  = fold over r of send[r][t][h], rounded to dtype (the reduce-scatter
 *           value);
 *   inv   = 1 / sqrt(mean over h of s[h]^2 + eps), computed in fp32;
 *   recv[q][t][h] = dtype(s[h] * inv * gamma[h]) for every q.
 * This equals reduce-scatter, RMSNorm on each owner's rows, then all-gather,
 * whenever each shard holds whole rows.  The sum of squares is accumulated in
 * fp32 in a fixed order for a given launch form (the split-row form adds
 * per-piece sums in piece order, the one-pass forms per-lane sums across the
 * row), so results are reproducible; against an exact norm the relative error
 * is at most about (hidden/2 + 4) * 2^-24 either way.
 * The split-row form (see ccl_launch_config_t) runs two kernels: the first
 * parks each row's folded values s in recv[0] (so recv[0] holds s, not the
 * result, until the second kernel has run) and writes one fp32 partial sum
 * per 4 KiB piece to scratch; the second scales and stores.  That scratch is
 * the calling stream's own device buffer, 4 bytes per piece: the first such
 * call on a (device, stream) allocates it with hipMalloc, a later call that
 * needs more allocates a larger one (at least twice the size), and every such
 * buffer is kept until the process ends.  A call made while its stream is
 * being captured cannot allocate: if the stream has no buffer large enough
 * yet, it runs the one-pass form instead, with the caller's stages and
 * occupancy where set (so make one eager call on the capturing stream first
 * to capture the split form).  A captured call keeps
 * the buffer of the stream it was captured on: replaying the graph while
 * other calls run on that stream, or on two streams at once, races.
 *
 *   dtype  CCL_FLOAT32, CCL_BFLOAT16 or CCL_FLOAT16 (op is sum).
 *   gamma  hidden elements of dtype, device memory, 16-byte aligned.
 *   eps    0 <= eps <= 1.
 *   Every send/recv buffer must be 16-byte aligned and hidden * element size
 *   a multiple of 16, with hidden * element size <= 32 KiB
 *   (else CCL_ERR_UNSUPPORTED).  In place recv[q] == send[q] is allowed.
 */
ccl_status_t ccl_all_reduce_rmsnorm(const void *const *send, void *const *recv, int nranks,
                                    size_t rows, size_t hidden, const void *gamma, float eps,
                                    int dtype, void *stream, const ccl_launch_config_t *cfg);

/*
 * ccl_all_reduce_rmsnorm for callers that cannot allocate device memory: code
 * under stream capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, checks and results as ccl_all_reduce_rmsnorm (the same
 * kernels, chosen by the same rules), but this call never allocates: the
 * split-row form's partial sums (4 bytes per 4 KiB piece of a row, rows x
 * ceil(hidden * element size / 4096) pieces) go to a fixed array of
 * CCL_NOALLOC_SCRATCH_BYTES in device memory that the library holds, one copy
 * per GPU, until the process ends.  A split-form call needing more returns
 * CCL_ERR_SCRATCH_LIMIT and launches nothing (with 16 KiB rows: up to 131,072
 * rows).  Every call on a GPU shares that GPU's array: calls that may overlap
 * on one GPU (other streams, graph replays) race and must be ordered by the
 * caller.  The array needs no clearing: a call reads only the sums its own
 * first kernel wrote.  The first call on a device looks up the array's device
 * address (hipGetSymbolAddress), which allocates nothing.
 */
ccl_status_t ccl_all_reduce_rmsnorm_noalloc(const void *const *send, void *const *recv,
                                            int nranks, size_t rows, size_t hidden,
                                            const void *gamma, float eps, int dtype, void *stream,
                                            const ccl_launch_config_t *cfg);

/*
 * Reduce ([roadmap] GENK section: ring reduce; [digest] s2.2: shard-in with a
 * single owner).  For i < count: recv[i] = fold over r of send[r][i].
 *
 *   send   P pointers, each to `count` elements.
 *   recv   the root's output buffer, `count` elements.
 *   root   the rank that owns recv, 0 <= root < P (it does not change the
 *          result: on one GPU every rank's buffer is addressable).
 *   In place: recv == send[r] is allowed (NCCL's in-place form is r = root);
 *   any other overlap gives CCL_ERR_ALIASING.
 */
ccl_status_t ccl_reduce(const void *const *send, void *recv, int nranks, size_t count, int dtype,
                        int op, int root, void *stream, const ccl_launch_config_t *cfg);

/*
 * Broadcast ([roadmap] GENK section: ring broadcast; [digest] s2.2: shard-out
 * from a single owner, one load serving every destination).  For q < P and
 * i < count: recv[q][i] = send[i].
 *
 *   send   the root's buffer, `count` elements.
 *   recv   P pointers, each to `count` elements.
 *   root   the rank that owns send, 0 <= root < P.
 *   In place: recv[q] == send is allowed (NCCL's form is q = root); other
 *   overlaps give CCL_ERR_ALIASING.  dtype only sets the element size.
 */
ccl_status_t ccl_broadcast(const void *send, void *const *recv, int nranks, size_t count,
                           int dtype, int root, void *stream, const ccl_launch_config_t *cfg);

/* ------------------------------------------------------------------ reshard
 * Layout-aware M-to-N reshard ([digest] s1.2 and s1.3): a tensor laid out
 * over a source mesh with one placement per mesh axis is moved to another
 * layout over a disjoint destination mesh.  Only the byte intervals each
 * destination rank needs are moved, found by intersecting index boxes; a
 * destination shard held by several replicas is read once and stored to all
 * of them (the single-GPU form of "one leader per domain, then local copies").
 */

typedef enum { CCL_REPLICATE = 0, CCL_SHARD = 1 } ccl_placement_kind_t;

/* Replicate(), or Shard(dim): dim is split into mesh-axis-size blocks of
 * ceil(D / axis size) indices each (the last ones short or empty). */
typedef struct {
    int32_t kind;
    int32_t dim;
} ccl_placement_t;

/* A mesh: ndims axes of the given sizes over the contiguous global ranks
 * start_rank .. start_rank + prod(dims) - 1, numbered row-major (last axis
 * fastest) -- the reading [digest] s1.4 Example A pins. */
typedef struct {
    int32_t ndims;
    int32_t start_rank;
    int64_t dims[CCL_MAX_MESH_DIMS];
} ccl_mesh_t;

/* The global tensor: row-major and contiguous on every rank. */
typedef struct {
    int32_t ndim;
    int32_t dtype; /* ccl_dtype_t; only its size matters to a copy */
    int64_t shape[CCL_MAX_TENSOR_DIMS];
} ccl_tensor_desc_t;

/* One planned byte interval (inspection only). */
typedef struct {
    int32_t src_rank;      /* global rank the bytes are read from (lowest source replica) */
    int32_t dst_shard;     /* destination shard index; its replicas all receive the bytes */
    int32_t leader;        /* global rank of the replica that leads this interval */
    int32_t num_replicas;  /* replicas of dst_shard */
    uint64_t src_offset;   /* byte offset in the source rank's local buffer */
    uint64_t dst_offset;   /* byte offset in every replica's local buffer */
    uint64_t length;       /* bytes */
} ccl_interval_t;

typedef struct ccl_plan ccl_plan_t;

/*
 * Plan a reshard on the host ([digest] s1.2: the transfer plan is derived from
 * the (mesh, placement) descriptors; intersecting intervals gives a
 * deterministic global plan with no over-delivery; leaders are picked so that
 * their loads differ by at most one).  Pure host code: no HIP call.
 *
 * Constraints ([digest] s1.3), each CCL_ERR_LAYOUT when broken: the meshes
 * are disjoint rank ranges; at most one mesh axis per layout is Shard; every
 * mesh has at most CCL_MAX_MESH_RANKS ranks.  Malformed descriptors give
 * CCL_ERR_INVALID_ARG.  Shard(dim) over an axis of m ranks cuts the dim into
 * blocks of ceil(D/m) indices; when m does not divide D the trailing blocks
 * are shorter or empty (the torch.chunk convention), so local buffer sizes
 * can differ between ranks (see ccl_plan_local_bytes).
 *
 * Intervals are maximal row-major runs, sorted by (dst_shard, dst_offset);
 * together they tile every destination shard exactly once.  *plan_out is
 * owned by the caller and released with ccl_plan_destroy.
 */
ccl_status_t ccl_reshard_plan(const ccl_tensor_desc_t *tensor, const ccl_mesh_t *src_mesh,
                              const ccl_placement_t *src_placements, const ccl_mesh_t *dst_mesh,
                              const ccl_placement_t *dst_placements, ccl_plan_t **plan_out);

/*
 * Execute a plan ([digest] s1.4, device data plane: each contribution enters
 * the destination shard once and is fanned out to the other replicas; here
 * one pass loads it once and stores it to every replica).
 *
 *   src_bufs   one pointer per source-mesh rank, in mesh order (rank
 *              start_rank + l at index l), each to that rank's local block.
 *   dst_bufs   one pointer per destination-mesh rank, likewise.
 *   Any overlap of two destination buffers, or of a source and a
 *   destination buffer, gives CCL_ERR_ALIASING.
 * The first call for a device and chunk size allocates the plan's device
 * interval table and a pinned host copy of it (hipMalloc, hipHostMalloc), and
 * uploads the table with an asynchronous copy on `stream`, ordered before the
 * copy kernel; the host does not wait.  The plan keeps both allocations until
 * ccl_plan_destroy.  A call on another stream while that upload may still be
 * in flight makes its stream wait for it (an event wait, not a host wait).
 * Because of the two allocations, make that first call outside stream
 * capture; later calls allocate nothing and can be captured.  The same holds
 * for ccl_reshard_copy_fp8, whose chunks are rounded to whole 128-element
 * blocks.
 */
ccl_status_t ccl_reshard_copy(const ccl_plan_t *plan, const void *const *src_bufs,
                              void *const *dst_bufs, void *stream,
                              const ccl_launch_config_t *cfg);

/*
 * Execute a plan with on-the-fly quantization in the staging pass (the
 * digest's M2N section lists quantizing weights inside the staging kernel as
 * future work and fixes no format; this is the format chosen here).  Every
 * destination buffer is written as OCP FP8 E4M3 codes (1 byte per element,
 * bias 7, largest finite 448) plus one fp32 scale per block of 128
 * consecutive elements of its local buffer: scale = amax / 448 in fp32 (1 when
 * that is zero: an all-zero block, or an amax so small that the quotient
 * underflows), code = round-to-nearest-even of x / scale in fp32,
 * saturated to +-448.  Dequantize as code_value * scale.  Source elements
 * must be finite: a block holding a NaN or an infinity gets unspecified
 * codes and scale.
 *
 *   src_bufs    as for ccl_reshard_copy (element type: fp32, bf16 or fp16).
 *   dst_codes   one pointer per destination-mesh rank, local-element-count
 *               bytes, 16-byte aligned.
 *   dst_scales  one pointer per destination-mesh rank, ceil(local elements /
 *               128) floats.
 * Returns CCL_ERR_UNSUPPORTED when the plan would split a 128-element
 * destination block across intervals or any interval offset is not 16-byte
 * aligned, and for an int32 plan.  Overlaps among the outputs or with a
 * source give CCL_ERR_ALIASING.
 */
ccl_status_t ccl_reshard_copy_fp8(const ccl_plan_t *plan, const void *const *src_bufs,
                                  void *const *dst_codes, float *const *dst_scales, void *stream,
                                  const ccl_launch_config_t *cfg);

/* Release a plan, its device tables and their pinned host copies (waiting
 * for a table upload still in flight).  Copy kernels that use the plan must
 * be complete. */
ccl_status_t ccl_plan_destroy(ccl_plan_t *plan);

/* Inspection: interval count, one interval, local buffer bytes of a mesh rank
 * (side 0 = source, 1 = destination; index = position in that mesh), the
 * replicas of a destination shard (global ranks, ascending), and the number
 * of distinct destination shards. */
ccl_status_t ccl_plan_num_intervals(const ccl_plan_t *plan, uint64_t *count);
ccl_status_t ccl_plan_get_interval(const ccl_plan_t *plan, uint64_t i, ccl_interval_t *out);
ccl_status_t ccl_plan_local_bytes(const ccl_plan_t *plan, int side, int index, uint64_t *bytes);
ccl_status_t ccl_plan_num_dst_shards(const ccl_plan_t *plan, int32_t *count);
ccl_status_t ccl_plan_shard_replicas(const ccl_plan_t *plan, int32_t dst_shard, int32_t *ranks,
                                     int32_t capacity, int32_t *count);

/* A static, human-readable name for a status code. */
const char *ccl_get_error_string(ccl_status_t status);

/* Library version as major*10000 + minor*100 + patch. */
int ccl_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CCL_H */
