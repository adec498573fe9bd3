/*
 * ccl_oracle.c -- plain, slow, obviously-correct CPU oracle for the collective
 * data plane.  TEST INFRASTRUCTURE ONLY: it is built and called by the test
 * suite, by the smoke check and by the bench's cpu_baseline leg, never by the
 * product library, and it shares no source, header, table or helper with it.
 *
 * Sources (the web pages this project is built from):
 *   [digest]  "NCCL M2N vs T-CCL" digest, lqnn.cn news 207677:
 *             s1.2 (layout-derived traffic, leader balance), s1.3 (Mesh /
 *             Shard / Replicate descriptors and their constraints), s1.4
 *             (Example A: TP4 -> TP2 x DP2, Example B: per-PP-stage reshard),
 *             s2.1 (add/min/max reduction op set), s2.2 (owner-local shard-in
 *             reduction, load-once shard-out), s2.3 (P shards for P ranks,
 *             NCCL-aligned collective semantics), s2.5 (all-reduce = shard-in
 *             followed by shard-out).
 *   [roadmap] "nccl-extensions" page (NCCL roadmap explainer), GENK section:
 *             ring all-reduce / reduce-scatter / all-gather semantics.
 *
 * Readings the pages leave open (each also listed in the design notes):
 *   - Reduction is a fold in rank order 0..P-1 that starts from rank 0's
 *     value, accumulates in fp32 (int32 wraps), and narrows once at the end.
 *   - bf16 and fp16 narrowing are round-to-nearest-even; a NaN becomes
 *     0x7FC0 (bf16) or 0x7E00 (fp16).
 *   - min keeps the earlier operand unless the later one is strictly smaller;
 *     max likewise with strictly greater (so ties, including +0/-0, keep the
 *     earlier rank's value).
 *   - Mesh ranks are numbered row-major (last mesh axis fastest) from
 *     start_rank; placements[k] applies to mesh axis k (both pinned by
 *     Example A in [digest] s1.4).
 *   - Shard(d) over m parts splits dim d into contiguous blocks of
 *     ceil(D/m) indices; the trailing blocks may be shorter or empty (the
 *     convention torch.chunk and DTensor use; the pages do not say).
 *
 * Every function returns 0 on success and a negative value on bad input.
 * Style: scalar loops, no SIMD intrinsics, no threads, no fast-math.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

/* The oracle's own type and op codes (the Python wrapper maps names to these). */
#define ORC_F32 0
#define ORC_BF16 1
#define ORC_I32 2
#define ORC_F16 3
#define ORC_SUM 0
#define ORC_MIN 1
#define ORC_MAX 2

#define ORC_MAX_MESH_DIMS 8
#define ORC_MAX_TENSOR_DIMS 8

/* ---------------------------------------------------------------- scalars */

static float bits_to_f32(uint32_t u) {
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t f32_to_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

/* bf16 -> fp32 is exact: the bf16 pattern is the top half of the fp32 one. */
static float orc_bf16_widen(uint16_t h) { return bits_to_f32((uint32_t)h << 16); }

/* fp32 -> bf16, round to nearest, ties to even. */
static uint16_t orc_bf16_narrow(float f) {
    uint32_t u = f32_to_bits(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)0x7fc0u; /* NaN */
    uint32_t lsb = (u >> 16) & 1u;
    u = u + 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

/* IEEE binary16 -> binary32 is exact (every half value is a float value). */
static float orc_f16_widen(uint16_t h) {
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
    if (e == 0x1f) return bits_to_f32(sign | 0x7f800000u | (m << 13)); /* inf / NaN */
    if (e != 0) return bits_to_f32(sign | ((e + 112u) << 23) | (m << 13));
    /* zero or subnormal: m * 2^-24, exact in fp32 */
    float v = (float)m * bits_to_f32(0x33800000u); /* 2^-24 */
    return sign ? -v : v;
}

/* binary32 -> binary16, round to nearest, ties to even; NaN -> 0x7e00. */
static uint16_t orc_f16_narrow(float f) {
    uint32_t u = f32_to_bits(f);
    uint32_t sign = (u >> 16) & 0x8000u;
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return (uint16_t)0x7e00u;
    if (a >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u); /* >= 65520 rounds to inf */
    if (a >= 0x38800000u) {                                  /* normal half: >= 2^-14 */
        uint32_t r = a + 0xfffu + ((a >> 13) & 1u);          /* round at bit 13 */
        r -= (uint32_t)(127 - 15) << 23;                     /* rebias the exponent */
        return (uint16_t)(sign | (r >> 13));
    }
    if (a <= 0x33000000u) return (uint16_t)sign; /* <= 2^-25 rounds to zero (tie to even) */
    /* subnormal half: k = value / 2^-24 = mant * 2^(e - 126), rounded to nearest even */
    uint32_t e = a >> 23;
    uint32_t mant = (a & 0x7fffffu) | 0x800000u;
    uint32_t s = 126u - e; /* 14 .. 24 */
    uint32_t k = (mant + (1u << (s - 1)) - 1u + ((mant >> s) & 1u)) >> s;
    return (uint16_t)(sign | k);
}

static int dtype_size(int dtype) {
    switch (dtype) {
    case ORC_F32: return 4;
    case ORC_BF16: return 2;
    case ORC_I32: return 4;
    case ORC_F16: return 2;
    default: return 0;
    }
}

static float fold_f32(float acc, float v, int op) {
    if (op == ORC_SUM) return acc + v;
    if (op == ORC_MIN) return (v < acc) ? v : acc;
    return (v > acc) ? v : acc;
}

static int32_t fold_i32(int32_t acc, int32_t v, int op) {
    if (op == ORC_SUM) return (int32_t)((uint32_t)acc + (uint32_t)v); /* wraps */
    if (op == ORC_MIN) return (v < acc) ? v : acc;
    return (v > acc) ? v : acc;
}

/*
 * The reduction of element i over the P rank buffers, written to dst
 * (one element of the given dtype).  Shard-in per [digest] s2.2: the owner
 * takes every rank's contribution and reduces it locally; the op set is the
 * one [digest] s2.1 lists (add, min, max).
 */
static void fold_element(const void *const *x, int P, int dtype, int op, size_t i, void *dst) {
    if (dtype == ORC_I32) {
        int32_t acc;
        memcpy(&acc, (const char *)x[0] + i * 4, 4);
        for (int r = 1; r < P; ++r) {
            int32_t v;
            memcpy(&v, (const char *)x[r] + i * 4, 4);
            acc = fold_i32(acc, v, op);
        }
        memcpy(dst, &acc, 4);
    } else if (dtype == ORC_F32) {
        float acc;
        memcpy(&acc, (const char *)x[0] + i * 4, 4);
        for (int r = 1; r < P; ++r) {
            float v;
            memcpy(&v, (const char *)x[r] + i * 4, 4);
            acc = fold_f32(acc, v, op);
        }
        memcpy(dst, &acc, 4);
    } else if (dtype == ORC_BF16) {
        uint16_t h;
        memcpy(&h, (const char *)x[0] + i * 2, 2);
        float acc = orc_bf16_widen(h);
        for (int r = 1; r < P; ++r) {
            memcpy(&h, (const char *)x[r] + i * 2, 2);
            acc = fold_f32(acc, orc_bf16_widen(h), op);
        }
        h = orc_bf16_narrow(acc);
        memcpy(dst, &h, 2);
    } else {
        uint16_t h;
        memcpy(&h, (const char *)x[0] + i * 2, 2);
        float acc = orc_f16_widen(h);
        for (int r = 1; r < P; ++r) {
            memcpy(&h, (const char *)x[r] + i * 2, 2);
            acc = fold_f32(acc, orc_f16_widen(h), op);
        }
        h = orc_f16_narrow(acc);
        memcpy(dst, &h, 2);
    }
}

static int check_common(const void *const *send, int P, int dtype, int op) {
    if (!send || P < 1 || dtype_size(dtype) == 0) return -1;
    if (op != ORC_SUM && op != ORC_MIN && op != ORC_MAX) return -1;
    return 0;
}

/* --------------------------------------------------------- collectives */

/*
 * All-reduce: every output buffer q receives, at every index i, the rank-order
 * fold of the P inputs at i.  [digest] s2.5 defines all-reduce as shard-in
 * followed by shard-out, so each of the P outputs holds the same reduced value.
 */
int orc_all_reduce(const void *const *send, void *const *recv, int P, size_t count, int dtype,
                   int op) {
    if (check_common(send, P, dtype, op) || !recv) return -1;
    const int s = dtype_size(dtype);
    char tmp[8];
    for (size_t i = 0; i < count; ++i) {
        fold_element(send, P, dtype, op, i, tmp);
        for (int q = 0; q < P; ++q) memcpy((char *)recv[q] + i * s, tmp, s);
    }
    return 0;
}

/*
 * Reduce-scatter: rank s keeps the reduction of shard s, i.e. input elements
 * [s*M, (s+1)*M) with M = recvcount ([digest] s2.3: the logical tensor is cut
 * into P shards, one per rank; s2.2: the owner reduces its shard locally).
 */
int orc_reduce_scatter(const void *const *send, void *const *recv, int P, size_t recvcount,
                       int dtype, int op) {
    if (check_common(send, P, dtype, op) || !recv) return -1;
    const int s = dtype_size(dtype);
    for (int sh = 0; sh < P; ++sh)
        for (size_t j = 0; j < recvcount; ++j)
            fold_element(send, P, dtype, op, (size_t)sh * recvcount + j,
                         (char *)recv[sh] + j * s);
    return 0;
}

/*
 * All-gather: every output q holds all shards in rank order, shard r at
 * element offset r*M ([digest] s2.2 shard-out: the owner's shard goes to every
 * peer).
 */
int orc_all_gather(const void *const *send, void *const *recv, int P, size_t sendcount,
                   int dtype) {
    if (!send || !recv || P < 1 || dtype_size(dtype) == 0) return -1;
    const size_t s = (size_t)dtype_size(dtype);
    for (int q = 0; q < P; ++q)
        for (int r = 0; r < P; ++r)
            for (size_t j = 0; j < sendcount; ++j)
                memcpy((char *)recv[q] + ((size_t)r * sendcount + j) * s,
                       (const char *)send[r] + j * s, s);
    return 0;
}

/*
 * Reduce: the single-owner form of the shard-in -- the root's buffer receives
 * the rank-order fold of all P inputs ([roadmap] GENK section: ring reduce;
 * [digest] s2.2: the owner reduces locally).
 */
int orc_reduce(const void *const *send, void *recv, int P, size_t count, int dtype, int op) {
    if (check_common(send, P, dtype, op) || !recv) return -1;
    const int s = dtype_size(dtype);
    for (size_t i = 0; i < count; ++i) fold_element(send, P, dtype, op, i, (char *)recv + i * s);
    return 0;
}

/*
 * Broadcast: the single-owner form of the shard-out -- every rank's buffer
 * receives the root's buffer ([roadmap] GENK section: ring broadcast;
 * [digest] s2.2: one load serves every destination).
 */
int orc_broadcast(const void *send, void *const *recv, int P, size_t count, int dtype) {
    if (!send || !recv || P < 1 || dtype_size(dtype) == 0) return -1;
    const size_t s = (size_t)dtype_size(dtype);
    for (int q = 0; q < P; ++q)
        for (size_t i = 0; i < count; ++i)
            memcpy((char *)recv[q] + i * s, (const char *)send + i * s, s);
    return 0;
}

/* One element of a float dtype as fp32 (exact). */
static float load_as_f32(const void *base, size_t i, int dtype) {
    if (dtype == ORC_F32) {
        float v;
        memcpy(&v, (const char *)base + i * 4, 4);
        return v;
    }
    uint16_t h;
    memcpy(&h, (const char *)base + i * 2, 2);
    return dtype == ORC_BF16 ? orc_bf16_widen(h) : orc_f16_widen(h);
}

static void store_from_f32(void *base, size_t i, int dtype, float v) {
    if (dtype == ORC_F32) {
        memcpy((char *)base + i * 4, &v, 4);
    } else {
        uint16_t h = dtype == ORC_BF16 ? orc_bf16_narrow(v) : orc_f16_narrow(v);
        memcpy((char *)base + i * 2, &h, 2);
    }
}

/*
 * All-reduce with RMSNorm fused between its two halves ([roadmap], the Device
 * API example that puts a Transformer RMSNorm between reduce-scatter and
 * all-gather in one kernel).  The tensor is rows x hidden on every rank.  Per
 * row t: s[h] = the rank-order fold of the P inputs, rounded to the dtype (the
 * value a reduce-scatter would hand over); then, in double precision,
 * inv = 1 / sqrt(mean_h s[h]^2 + eps) and y[h] = s[h] * inv * gamma[h],
 * rounded to fp32 and then to the dtype; every output q receives y.
 */
int orc_all_reduce_rmsnorm(const void *const *send, void *const *recv, int P, size_t rows,
                           size_t hidden, const void *gamma, double eps, int dtype) {
    if (check_common(send, P, dtype, ORC_SUM) || !recv || !gamma || dtype == ORC_I32) return -1;
    if (hidden == 0) return rows == 0 ? 0 : -1;
    char tmp[8];
    double ss;
    for (size_t t = 0; t < rows; ++t) {
        ss = 0.0;
        for (size_t h = 0; h < hidden; ++h) {
            fold_element(send, P, dtype, ORC_SUM, t * hidden + h, tmp);
            double v = (double)load_as_f32(tmp, 0, dtype);
            ss += v * v;
        }
        const double inv = 1.0 / sqrt(ss / (double)hidden + eps);
        for (size_t h = 0; h < hidden; ++h) {
            fold_element(send, P, dtype, ORC_SUM, t * hidden + h, tmp);
            const double v = (double)load_as_f32(tmp, 0, dtype);
            const double g = (double)load_as_f32(gamma, h, dtype);
            const float y = (float)(v * inv * g);
            for (int q = 0; q < P; ++q) store_from_f32(recv[q], t * hidden + h, dtype, y);
        }
    }
    return 0;
}

/* The fold at selected indices only: out[k] = fold(idx[k]).  Lets a test check
 * outputs of buffers far too large for the full oracle. */
int orc_fold_at(const void *const *send, int P, int dtype, int op, const uint64_t *idx, size_t n,
                void *out) {
    if (check_common(send, P, dtype, op) || (n && (!idx || !out))) return -1;
    const int s = dtype_size(dtype);
    for (size_t k = 0; k < n; ++k) fold_element(send, P, dtype, op, (size_t)idx[k], (char *)out + k * s);
    return 0;
}

/* ------------------------------------------------------------- reshard */

/* A layout: a mesh of ranks plus one placement per mesh axis ([digest] s1.3). */
typedef struct {
    int ndims;
    int64_t dims[ORC_MAX_MESH_DIMS];
    int64_t start_rank;
    int kind[ORC_MAX_MESH_DIMS]; /* 0 = Replicate, 1 = Shard */
    int sdim[ORC_MAX_MESH_DIMS]; /* tensor dim for Shard */
} orc_layout;

static int64_t layout_size(const orc_layout *L) {
    int64_t n = 1;
    for (int k = 0; k < L->ndims; ++k) n *= L->dims[k];
    return n;
}

static int layout_check(const orc_layout *L, int ndim, const int64_t *shape) {
    (void)shape; /* any dim size is valid: uneven blocks are clipped */
    if (L->ndims < 1 || L->ndims > ORC_MAX_MESH_DIMS || L->start_rank < 0) return -1;
    for (int k = 0; k < L->ndims; ++k) {
        if (L->dims[k] < 1) return -1;
        if (L->kind[k] == 1) {
            int d = L->sdim[k];
            if (d < 0 || d >= ndim) return -1;
            for (int k2 = 0; k2 < k; ++k2)
                if (L->kind[k2] == 1 && L->sdim[k2] == d) return -1; /* same dim twice */
        } else if (L->kind[k] != 0) {
            return -1;
        }
    }
    return 0;
}

/* Mesh coordinate of the l-th rank of the mesh: row-major, last axis fastest. */
static void unravel_mesh(const orc_layout *L, int64_t l, int64_t *c) {
    for (int k = L->ndims - 1; k >= 0; --k) {
        c[k] = l % L->dims[k];
        l /= L->dims[k];
    }
}

/* The index box [lo, hi) a mesh coordinate holds: Shard(d) on axis k cuts dim d
 * into blocks of ceil(D / dims[k]) indices and takes block c[k] (clipped to D,
 * so late blocks can be short or empty); Replicate leaves the dim whole. */
static void rank_box(const orc_layout *L, const int64_t *c, int ndim, const int64_t *shape,
                     int64_t *lo, int64_t *hi) {
    for (int d = 0; d < ndim; ++d) {
        lo[d] = 0;
        hi[d] = shape[d];
    }
    for (int k = 0; k < L->ndims; ++k) {
        if (L->kind[k] != 1) continue;
        int d = L->sdim[k];
        int64_t part = (shape[d] + L->dims[k] - 1) / L->dims[k];
        lo[d] = c[k] * part < shape[d] ? c[k] * part : shape[d];
        hi[d] = lo[d] + part < shape[d] ? lo[d] + part : shape[d];
    }
}

static int box_contains(const int64_t *lo, const int64_t *hi, const int64_t *g, int ndim) {
    for (int d = 0; d < ndim; ++d)
        if (g[d] < lo[d] || g[d] >= hi[d]) return 0;
    return 1;
}

/* Row-major offset of g inside the box. */
static int64_t box_offset(const int64_t *lo, const int64_t *hi, const int64_t *g, int ndim) {
    int64_t off = 0;
    for (int d = 0; d < ndim; ++d) off = off * (hi[d] - lo[d]) + (g[d] - lo[d]);
    return off;
}

static int fill_layout(orc_layout *L, int ndims, const int64_t *dims, int64_t start,
                       const int *kind, const int *sdim) {
    if (ndims < 1 || ndims > ORC_MAX_MESH_DIMS || !dims || !kind || !sdim) return -1;
    L->ndims = ndims;
    L->start_rank = start;
    for (int k = 0; k < ndims; ++k) {
        L->dims[k] = dims[k];
        L->kind[k] = kind[k];
        L->sdim[k] = sdim[k];
    }
    return 0;
}

static int meshes_disjoint(const orc_layout *A, const orc_layout *B) {
    int64_t a0 = A->start_rank, a1 = a0 + layout_size(A);
    int64_t b0 = B->start_rank, b1 = b0 + layout_size(B);
    return a1 <= b0 || b1 <= a0;
}

/*
 * Reshard by brute force, one element at a time ([digest] s1.2: only the bytes
 * the destination layout needs are moved; s1.3: layouts are (mesh, placement)
 * pairs; the two meshes must be disjoint).
 *
 * For every global index g: the source ranks whose box contains g all hold the
 * same value (checked); the value is taken from the lowest such rank and
 * written into every destination rank whose box contains g, at g's row-major
 * offset inside that rank's box.  src_bufs[l] / dst_bufs[l] belong to the l-th
 * rank of the respective mesh.  Returns -3 if source replicas disagree and -4
 * if some destination element is not covered.
 */
int orc_reshard(int ndim, const int64_t *shape, int elem_size,
                int s_ndims, const int64_t *s_dims, int64_t s_start, const int *s_kind,
                const int *s_sdim,
                int d_ndims, const int64_t *d_dims, int64_t d_start, const int *d_kind,
                const int *d_sdim,
                const void *const *src_bufs, void *const *dst_bufs) {
    orc_layout S, D;
    if (ndim < 1 || ndim > ORC_MAX_TENSOR_DIMS || !shape || elem_size < 1 || elem_size > 16)
        return -1;
    for (int d = 0; d < ndim; ++d)
        if (shape[d] < 0) return -1;
    if (fill_layout(&S, s_ndims, s_dims, s_start, s_kind, s_sdim)) return -1;
    if (fill_layout(&D, d_ndims, d_dims, d_start, d_kind, d_sdim)) return -1;
    int rc;
    if ((rc = layout_check(&S, ndim, shape))) return rc;
    if ((rc = layout_check(&D, ndim, shape))) return rc;
    if (!meshes_disjoint(&S, &D)) return -1;
    if (!src_bufs || !dst_bufs) return -1;

    int64_t numel = 1;
    for (int d = 0; d < ndim; ++d) numel *= shape[d];
    const int64_t ns = layout_size(&S), nd = layout_size(&D);
    int64_t g[ORC_MAX_TENSOR_DIMS], c[ORC_MAX_MESH_DIMS];
    int64_t lo[ORC_MAX_TENSOR_DIMS], hi[ORC_MAX_TENSOR_DIMS];

    for (int64_t flat = 0; flat < numel; ++flat) {
        int64_t t = flat;
        for (int d = ndim - 1; d >= 0; --d) {
            g[d] = t % shape[d];
            t /= shape[d];
        }
        const unsigned char *val = NULL;
        for (int64_t l = 0; l < ns; ++l) {
            unravel_mesh(&S, l, c);
            rank_box(&S, c, ndim, shape, lo, hi);
            if (!box_contains(lo, hi, g, ndim)) continue;
            const unsigned char *p =
                (const unsigned char *)src_bufs[l] + box_offset(lo, hi, g, ndim) * elem_size;
            if (!val)
                val = p;
            else if (memcmp(val, p, (size_t)elem_size) != 0)
                return -3;
        }
        if (!val) return -4; /* cannot happen for a valid layout */
        int written = 0;
        for (int64_t l = 0; l < nd; ++l) {
            unravel_mesh(&D, l, c);
            rank_box(&D, c, ndim, shape, lo, hi);
            if (!box_contains(lo, hi, g, ndim)) continue;
            memcpy((unsigned char *)dst_bufs[l] + box_offset(lo, hi, g, ndim) * elem_size, val,
                   (size_t)elem_size);
            ++written;
        }
        if (!written) return -4;
    }
    return 0;
}

/*
 * Point query of the same reshard: for destination rank dst_l (its index in
 * the destination mesh) and element offsets local[k] inside its buffer, write
 * the value that rank must end up holding.  The offset is mapped back to its
 * global index through the rank's box, and the value is read from the lowest
 * source rank whose box holds that index.
 */
int orc_reshard_at(int ndim, const int64_t *shape, int elem_size,
                   int s_ndims, const int64_t *s_dims, int64_t s_start, const int *s_kind,
                   const int *s_sdim,
                   int d_ndims, const int64_t *d_dims, int64_t d_start, const int *d_kind,
                   const int *d_sdim,
                   const void *const *src_bufs, int64_t dst_l, const uint64_t *local, size_t n,
                   void *out) {
    orc_layout S, D;
    if (ndim < 1 || ndim > ORC_MAX_TENSOR_DIMS || !shape || elem_size < 1 || elem_size > 16)
        return -1;
    if (fill_layout(&S, s_ndims, s_dims, s_start, s_kind, s_sdim)) return -1;
    if (fill_layout(&D, d_ndims, d_dims, d_start, d_kind, d_sdim)) return -1;
    int rc;
    if ((rc = layout_check(&S, ndim, shape))) return rc;
    if ((rc = layout_check(&D, ndim, shape))) return rc;
    if (dst_l < 0 || dst_l >= layout_size(&D) || !src_bufs || (n && (!local || !out))) return -1;

    int64_t c[ORC_MAX_MESH_DIMS], lo[ORC_MAX_TENSOR_DIMS], hi[ORC_MAX_TENSOR_DIMS];
    int64_t dlo[ORC_MAX_TENSOR_DIMS], dhi[ORC_MAX_TENSOR_DIMS], g[ORC_MAX_TENSOR_DIMS];
    unravel_mesh(&D, dst_l, c);
    rank_box(&D, c, ndim, shape, dlo, dhi);
    int64_t local_numel = 1;
    for (int d = 0; d < ndim; ++d) local_numel *= dhi[d] - dlo[d];
    const int64_t ns = layout_size(&S);

    for (size_t k = 0; k < n; ++k) {
        if ((int64_t)local[k] >= local_numel) return -1;
        int64_t t = (int64_t)local[k];
        for (int d = ndim - 1; d >= 0; --d) {
            int64_t ext = dhi[d] - dlo[d];
            g[d] = dlo[d] + t % ext;
            t /= ext;
        }
        int found = 0;
        for (int64_t l = 0; l < ns && !found; ++l) {
            unravel_mesh(&S, l, c);
            rank_box(&S, c, ndim, shape, lo, hi);
            if (!box_contains(lo, hi, g, ndim)) continue;
            memcpy((unsigned char *)out + k * (size_t)elem_size,
                   (const unsigned char *)src_bufs[l] + box_offset(lo, hi, g, ndim) * elem_size,
                   (size_t)elem_size);
            found = 1;
        }
        if (!found) return -4;
    }
    return 0;
}

/* ------------------------------------------------- fp8 staging quantization */

/*
 * OCP FP8 E4M3 ("e4m3fn": 1 sign, 4 exponent bits with bias 7, 3 mantissa
 * bits, no infinities, S.1111.111 is NaN, largest finite 448): the value of a
 * code, straight from that definition.
 */
static double e4m3_value(unsigned code) {
    const unsigned e = (code >> 3) & 15u, m = code & 7u;
    double v = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, (int)e - 7);
    return (code & 0x80u) ? -v : v;
}

/*
 * Nearest E4M3 code to y, ties to the code with an even mantissa, magnitudes
 * above 448 saturated to 448 (a brute-force search over the 127 finite
 * non-negative codes).  The sign of y (including -0) is kept.
 */
static unsigned e4m3_nearest_sat(float y) {
    const double a = fabs((double)y);
    const unsigned sign = signbit(y) ? 0x80u : 0u;
    if (a >= 448.0) return sign | 0x7eu;
    unsigned best = 0;
    double best_d = a;
    for (unsigned c = 1; c < 0x7f; ++c) {
        const double d = fabs(e4m3_value(c) - a);
        if (d < best_d || (d == best_d && (c & 1u) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return sign | best;
}

/*
 * Quantize n elements in blocks of `block`: per block, amax = max |x| (fp32),
 * scale = amax / 448 in fp32 (1 when that is 0: an all-zero block, or an amax
 * so small that the quotient underflows), code = nearest E4M3 to
 * x / scale in fp32.  The M2N part of the digest (lqnn.cn news 207677) s1.5
 * names quantizing weights on the fly inside the staging kernel as future
 * work without fixing a format; this is the format this library picks.
 */
int orc_quantize_e4m3(const void *x, int dtype, size_t n, size_t block, uint8_t *codes,
                      float *scales) {
    if (!x || dtype == ORC_I32 || dtype_size(dtype) == 0 || block == 0 || (n && (!codes || !scales)))
        return -1;
    for (size_t b0 = 0; b0 < n; b0 += block) {
        const size_t b1 = b0 + block < n ? b0 + block : n;
        float amax = 0.f;
        for (size_t i = b0; i < b1; ++i) {
            const float v = fabsf(load_as_f32(x, i, dtype));
            if (v > amax) amax = v;
        }
        const float q = amax / 448.0f;
        const float scale = q > 0.f ? q : 1.0f;
        scales[b0 / block] = scale;
        for (size_t i = b0; i < b1; ++i) codes[i] = (uint8_t)e4m3_nearest_sat(load_as_f32(x, i, dtype) / scale);
    }
    return 0;
}

double orc_e4m3_value(unsigned code) { return e4m3_value(code); }
unsigned orc_e4m3_nearest_sat(float y) { return e4m3_nearest_sat(y); }

/* Number of elements the l-th rank of a layout holds (its box volume). */
int64_t orc_local_numel(int ndim, const int64_t *shape, int m_ndims, const int64_t *m_dims,
                        const int *kind, const int *sdim, int64_t l) {
    orc_layout L;
    if (ndim < 1 || ndim > ORC_MAX_TENSOR_DIMS || !shape) return -1;
    if (fill_layout(&L, m_ndims, m_dims, 0, kind, sdim)) return -1;
    if (layout_check(&L, ndim, shape)) return -1;
    if (l < 0 || l >= layout_size(&L)) return -1;
    int64_t c[ORC_MAX_MESH_DIMS], lo[ORC_MAX_TENSOR_DIMS], hi[ORC_MAX_TENSOR_DIMS];
    unravel_mesh(&L, l, c);
    rank_box(&L, c, ndim, shape, lo, hi);
    int64_t n = 1;
    for (int d = 0; d < ndim; ++d) n *= hi[d] - lo[d];
    return n;
}

/* Exposed for tests of the rounding rules themselves. */
uint16_t orc_narrow_bf16(float f) { return orc_bf16_narrow(f); }
float orc_widen_bf16(uint16_t h) { return orc_bf16_widen(h); }
uint16_t orc_narrow_f16(float f) { return orc_f16_narrow(f); }
float orc_widen_f16(uint16_t h) { return orc_f16_widen(h); }
