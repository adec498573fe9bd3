// Reshard planner: byte-interval intersection of two (mesh, placement)
// layouts, on the host.  Follows the M2N description in the "NCCL M2N vs
// T-CCL" digest (lqnn.cn news 207677): s1.2 (the plan is derived from the
// descriptors, only intersecting intervals are moved, leaders are balanced),
// s1.3 (Mesh / Shard / Replicate and the layout constraints).
//
// A layout with Shard(d) on mesh axis k splits tensor dim d into blocks of
// ceil(D / dims[k]) indices, clipped to D so trailing blocks may be short or
// empty (the torch.chunk convention; the pages leave uneven splits open);
// mesh rank l (row-major coordinates c) holds block c[k] and is a replica of
// every other rank with the same c[k].  With no Shard axis, every
// rank holds the whole tensor.  Each distinct block ("shard") is a box of
// global indices; the plan intersects every destination shard with every
// source shard and emits the intersection as maximal runs that are
// contiguous in both local row-major layouts.
#include <algorithm>
#include <cstdint>
#include <new>
#include <vector>

#include "ccl_internal.h"

namespace {

constexpr uint64_t kMaxIntervals = uint64_t(1) << 24;

struct Layout {
  int nd;                 // mesh axes
  int64_t dims[CCL_MAX_MESH_DIMS];
  int start;
  int size;               // ranks
  int shard_axis;         // -1 = fully replicated
  int shard_dim;          // tensor dim split by shard_axis
  int64_t parts;          // blocks along shard_dim (1 if replicated)
};

ccl_status_t make_layout(const ccl_mesh_t *m, const ccl_placement_t *pl, int ndim, Layout *L) {
  if (!m || !pl) return CCL_ERR_INVALID_ARG;
  if (m->ndims < 1 || m->ndims > CCL_MAX_MESH_DIMS || m->start_rank < 0)
    return CCL_ERR_INVALID_ARG;
  L->nd = m->ndims;
  L->start = m->start_rank;
  int64_t size = 1;
  for (int k = 0; k < m->ndims; ++k) {
    if (m->dims[k] < 1) return CCL_ERR_INVALID_ARG;
    L->dims[k] = m->dims[k];
    size *= m->dims[k];
    if (size > CCL_MAX_MESH_RANKS) return CCL_ERR_LAYOUT;
  }
  if ((int64_t)m->start_rank + size > INT32_MAX) return CCL_ERR_INVALID_ARG;
  L->size = (int)size;
  L->shard_axis = -1;
  L->shard_dim = 0;
  L->parts = 1;
  for (int k = 0; k < m->ndims; ++k) {
    if (pl[k].kind == CCL_REPLICATE) continue;
    if (pl[k].kind != CCL_SHARD) return CCL_ERR_INVALID_ARG;
    if (pl[k].dim < 0 || pl[k].dim >= ndim) return CCL_ERR_INVALID_ARG;
    if (L->shard_axis >= 0) return CCL_ERR_LAYOUT;  // at most one sharded mesh axis
    L->shard_axis = k;
    L->shard_dim = pl[k].dim;
    L->parts = m->dims[k];
  }
  return CCL_OK;
}

// Coordinate of mesh rank l along the shard axis (row-major, last axis fastest).
int64_t shard_of(const Layout &L, int l) {
  if (L.shard_axis < 0) return 0;
  int64_t stride = 1;
  for (int k = L.nd - 1; k > L.shard_axis; --k) stride *= L.dims[k];
  return (l / stride) % L.dims[L.shard_axis];
}

void shard_box(const Layout &L, int64_t t, int ndim, const int64_t *shape, int64_t *lo,
               int64_t *hi) {
  for (int d = 0; d < ndim; ++d) {
    lo[d] = 0;
    hi[d] = shape[d];
  }
  if (L.shard_axis >= 0) {
    const int64_t D = shape[L.shard_dim];
    const int64_t part = (D + L.parts - 1) / L.parts;
    lo[L.shard_dim] = std::min(t * part, D);
    hi[L.shard_dim] = std::min(lo[L.shard_dim] + part, D);
  }
}

uint64_t box_volume(const int64_t *lo, const int64_t *hi, int ndim) {
  uint64_t n = 1;
  for (int d = 0; d < ndim; ++d) n *= (uint64_t)(hi[d] - lo[d]);
  return n;
}

int64_t rowmajor_offset(const int64_t *g, const int64_t *lo, const int64_t *hi, int ndim) {
  int64_t off = 0;
  for (int d = 0; d < ndim; ++d) off = off * (hi[d] - lo[d]) + (g[d] - lo[d]);
  return off;
}

}  // namespace

extern "C" {

ccl_status_t ccl_reshard_plan(const ccl_tensor_desc_t *tensor, const ccl_mesh_t *src_mesh,
                              const ccl_placement_t *src_placements, const ccl_mesh_t *dst_mesh,
                              const ccl_placement_t *dst_placements, ccl_plan_t **plan_out) {
  if (!tensor || !plan_out) return CCL_ERR_INVALID_ARG;
  *plan_out = nullptr;
  const int ndim = tensor->ndim;
  if (ndim < 1 || ndim > CCL_MAX_TENSOR_DIMS) return CCL_ERR_INVALID_ARG;
  const int esz = ccl::dtype_size(tensor->dtype);
  if (!esz) return CCL_ERR_INVALID_ARG;
  uint64_t numel = 1;
  for (int d = 0; d < ndim; ++d) {
    if (tensor->shape[d] < 0) return CCL_ERR_INVALID_ARG;
    if (tensor->shape[d] && numel > (UINT64_MAX / 16) / (uint64_t)tensor->shape[d])
      return CCL_ERR_INVALID_ARG;
    numel *= (uint64_t)tensor->shape[d];
  }
  const int64_t *shape = tensor->shape;
  Layout S, D;
  ccl_status_t st;
  if ((st = make_layout(src_mesh, src_placements, ndim, &S))) return st;
  if ((st = make_layout(dst_mesh, dst_placements, ndim, &D))) return st;
  // The two meshes must be disjoint rank ranges.
  if (!(S.start + S.size <= D.start || D.start + D.size <= S.start)) return CCL_ERR_LAYOUT;

  ccl_plan *p = new (std::nothrow) ccl_plan();
  if (!p) return CCL_ERR_NOMEM;
  p->elem_size = esz;
  p->dtype = tensor->dtype;
  p->src_start = S.start;
  p->dst_start = D.start;
  p->n_src = S.size;
  p->n_dst = D.size;
  p->n_dst_shards = (int32_t)D.parts;

  int64_t blo[CCL_MAX_TENSOR_DIMS], bhi[CCL_MAX_TENSOR_DIMS];
  p->src_local_bytes.resize(S.size);
  for (int l = 0; l < S.size; ++l) {
    shard_box(S, shard_of(S, l), ndim, shape, blo, bhi);
    p->src_local_bytes[l] = box_volume(blo, bhi, ndim) * esz;
  }
  p->dst_local_bytes.resize(D.size);
  for (int l = 0; l < D.size; ++l) {
    shard_box(D, shard_of(D, l), ndim, shape, blo, bhi);
    p->dst_local_bytes[l] = box_volume(blo, bhi, ndim) * esz;
  }

  // Source holder of each source shard: its lowest rank (all replicas agree).
  std::vector<int32_t> src_holder(S.parts, -1);
  for (int l = 0; l < S.size; ++l) {
    int64_t t = shard_of(S, l);
    if (src_holder[t] < 0) src_holder[t] = l;
  }
  p->replicas.assign(D.parts, {});
  for (int l = 0; l < D.size; ++l) p->replicas[shard_of(D, l)].push_back(l);

  int64_t slo[CCL_MAX_TENSOR_DIMS], shi[CCL_MAX_TENSOR_DIMS];
  int64_t dlo[CCL_MAX_TENSOR_DIMS], dhi[CCL_MAX_TENSOR_DIMS];
  int64_t lo[CCL_MAX_TENSOR_DIMS], hi[CCL_MAX_TENSOR_DIMS], g[CCL_MAX_TENSOR_DIMS];
  if (numel > 0) {
    for (int64_t td = 0; td < D.parts; ++td) {
      shard_box(D, td, ndim, shape, dlo, dhi);
      const size_t first = p->intervals.size();
      for (int64_t ts = 0; ts < S.parts; ++ts) {
        shard_box(S, ts, ndim, shape, slo, shi);
        bool empty = false;
        for (int d = 0; d < ndim; ++d) {
          lo[d] = std::max(slo[d], dlo[d]);
          hi[d] = std::min(shi[d], dhi[d]);
          if (lo[d] >= hi[d]) empty = true;
        }
        if (empty) continue;
        // Trailing dims that are whole in the intersection and in both local
        // boxes merge into one run with the first dim that is not.
        int k = ndim - 1;
        while (k > 0 && hi[k] - lo[k] == shi[k] - slo[k] && hi[k] - lo[k] == dhi[k] - dlo[k]) --k;
        uint64_t run = 1;
        for (int d = k; d < ndim; ++d) run *= (uint64_t)(hi[d] - lo[d]);
        uint64_t nruns = 1;
        for (int d = 0; d < k; ++d) nruns *= (uint64_t)(hi[d] - lo[d]);
        if (p->intervals.size() + nruns > kMaxIntervals) {
          delete p;
          return CCL_ERR_UNSUPPORTED;
        }
        for (uint64_t o = 0; o < nruns; ++o) {
          uint64_t t = o;
          for (int d = k - 1; d >= 0; --d) {
            const uint64_t ext = (uint64_t)(hi[d] - lo[d]);
            g[d] = lo[d] + (int64_t)(t % ext);
            t /= ext;
          }
          for (int d = k; d < ndim; ++d) g[d] = lo[d];
          ccl::PlanInterval iv;
          iv.src_local = src_holder[ts];
          iv.dst_shard = (int32_t)td;
          iv.leader = -1;
          iv.src_off = (uint64_t)rowmajor_offset(g, slo, shi, ndim) * esz;
          iv.dst_off = (uint64_t)rowmajor_offset(g, dlo, dhi, ndim) * esz;
          iv.len = run * esz;
          p->intervals.push_back(iv);
        }
      }
      // Deterministic order inside the shard, then balanced leaders: the j-th
      // interval of a shard is led by replica j mod rho.
      std::sort(p->intervals.begin() + first, p->intervals.end(),
                [](const ccl::PlanInterval &a, const ccl::PlanInterval &b) {
                  return a.dst_off < b.dst_off;
                });
      const auto &rep = p->replicas[td];
      for (size_t j = first; j < p->intervals.size(); ++j)
        p->intervals[j].leader = D.start + rep[(j - first) % rep.size()];
    }
  }
  const uint64_t block_bytes = 128 * (uint64_t)esz;
  for (const auto &iv : p->intervals) {
    if (iv.src_off % 16 || iv.dst_off % 16) p->offsets_aligned16 = false;
    if (iv.dst_off % 256) p->dst_offsets_aligned256 = false;
    const uint64_t end = iv.dst_off + iv.len;
    const uint64_t local = p->dst_local_bytes[p->replicas[iv.dst_shard][0]];
    if (iv.dst_off % block_bytes || (end % block_bytes && end != local)) p->fp8_blocks_ok = false;
  }
  *plan_out = p;
  return CCL_OK;
}

ccl_status_t ccl_plan_destroy(ccl_plan_t *plan) {
  if (!plan) return CCL_ERR_INVALID_ARG;
  ccl::reshard_release(plan);
  delete plan;
  return CCL_OK;
}

ccl_status_t ccl_plan_num_intervals(const ccl_plan_t *plan, uint64_t *count) {
  if (!plan || !count) return CCL_ERR_INVALID_ARG;
  *count = plan->intervals.size();
  return CCL_OK;
}

ccl_status_t ccl_plan_get_interval(const ccl_plan_t *plan, uint64_t i, ccl_interval_t *out) {
  if (!plan || !out || i >= plan->intervals.size()) return CCL_ERR_INVALID_ARG;
  const ccl::PlanInterval &iv = plan->intervals[i];
  out->src_rank = plan->src_start + iv.src_local;
  out->dst_shard = iv.dst_shard;
  out->leader = iv.leader;
  out->num_replicas = (int32_t)plan->replicas[iv.dst_shard].size();
  out->src_offset = iv.src_off;
  out->dst_offset = iv.dst_off;
  out->length = iv.len;
  return CCL_OK;
}

ccl_status_t ccl_plan_local_bytes(const ccl_plan_t *plan, int side, int index, uint64_t *bytes) {
  if (!plan || !bytes || (side != 0 && side != 1)) return CCL_ERR_INVALID_ARG;
  const auto &v = side == 0 ? plan->src_local_bytes : plan->dst_local_bytes;
  if (index < 0 || index >= (int)v.size()) return CCL_ERR_INVALID_ARG;
  *bytes = v[index];
  return CCL_OK;
}

ccl_status_t ccl_plan_num_dst_shards(const ccl_plan_t *plan, int32_t *count) {
  if (!plan || !count) return CCL_ERR_INVALID_ARG;
  *count = plan->n_dst_shards;
  return CCL_OK;
}

ccl_status_t ccl_plan_shard_replicas(const ccl_plan_t *plan, int32_t dst_shard, int32_t *ranks,
                                     int32_t capacity, int32_t *count) {
  if (!plan || !count || dst_shard < 0 || dst_shard >= plan->n_dst_shards)
    return CCL_ERR_INVALID_ARG;
  const auto &rep = plan->replicas[dst_shard];
  *count = (int32_t)rep.size();
  if (capacity < (int32_t)rep.size() || (!ranks && !rep.empty())) return CCL_ERR_INVALID_ARG;
  for (size_t j = 0; j < rep.size(); ++j) ranks[j] = plan->dst_start + rep[j];
  return CCL_OK;
}

}  // extern "C"
