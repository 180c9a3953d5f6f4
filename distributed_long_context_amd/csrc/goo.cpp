// GOO step planner on the host.  [Mesh] section 3.4 (2-D Greedy Overlapping
// Optimization); the rules and the readings are stated with the declaration of
// mesh_attn_goo_plan.  State is kept in bit sets over the at most 16 compute
// tasks, so a step costs O(k_q k_kv) and the planner allocates nothing.
#include <cmath>
#include <cstdint>
#include <cstring>

#include "mesh_attn.h"
#include "ma_internal.h"

using namespace ma;

extern "C" int32_t mesh_attn_goo_plan(int32_t kq, int32_t kkv, double t_agq, double t_agkv, double t_rsq,
                                      const double* t_c, double gamma, int32_t max_steps, ma_goo_step* steps) {
  if (kq < 1 || kkv < 1 || kq * kkv > MA_GOO_MAX_COMPUTE || !t_c || !steps)
    return -set_error(MA_ERR_INVALID, "goo_plan: need k_q, k_kv >= 1, k_q * k_kv <= 16 and non-null arrays");
  if (!(t_agq > 0) || !(t_agkv > 0) || !(t_rsq > 0) || !std::isfinite(t_agq) || !std::isfinite(t_agkv) ||
      !std::isfinite(t_rsq) || !(gamma >= 0) || !std::isfinite(gamma))
    return -set_error(MA_ERR_INVALID, "goo_plan: communication times must be > 0 and gamma >= 0, all finite");
  const int nc = kq * kkv;
  for (int c = 0; c < nc; ++c)
    if (!(t_c[c] >= 0) || !std::isfinite(t_c[c])) return -set_error(MA_ERR_INVALID, "goo_plan: bad compute time");
  if (max_steps < 2 * kq + kkv + nc) return -set_error(MA_ERR_INVALID, "goo_plan: max_steps below 2 k_q + k_kv + k_q k_kv");

  uint32_t agq_done = 0, agkv_done = 0, rs_done = 0;  // bit i / j: chunk collective finished
  uint32_t c_done = 0;                                 // bit i * kkv + j: compute task finished
  // compute tasks whose two inputs have arrived, given the AG bit sets
  auto ready_set = [&](uint32_t q, uint32_t k) {
    uint32_t r = 0;
    for (int i = 0; i < kq; ++i)
      if (q >> i & 1u)
        for (int j = 0; j < kkv; ++j)
          if (k >> j & 1u) r |= 1u << (i * kkv + j);
    return r;
  };
  auto row_mask = [&](int i) { return ((1u << kkv) - 1u) << (i * kkv); };
  auto lowest_unset = [](uint32_t bits, int n) {
    for (int x = 0; x < n; ++x)
      if (!(bits >> x & 1u)) return x;
    return -1;
  };
  auto time_of = [&](uint32_t set) {  // summed in (i, j) order
    double t = 0.0;
    for (int c = 0; c < nc; ++c)
      if (set >> c & 1u) t += t_c[c];
    return t;
  };

  int ns = 0;
  for (;;) {
    const uint32_t avail = ready_set(agq_done, agkv_done) & ~c_done;
    // candidates in tie-break order: AG-KV, AG-Q, RS-Q
    int type = MA_GOO_NONE, index = 0;
    double best = -1.0;
    const int jk = lowest_unset(agkv_done, kkv);
    if (jk >= 0) {
      const double p = time_of(ready_set(agq_done, agkv_done | 1u << jk) & ~ready_set(agq_done, agkv_done) & ~c_done) / t_agkv;
      if (p > best) { best = p; type = MA_GOO_AG_KV; index = jk; }
    }
    const int iq = lowest_unset(agq_done, kq);
    if (iq >= 0) {
      const double p = time_of(ready_set(agq_done | 1u << iq, agkv_done) & ~ready_set(agq_done, agkv_done) & ~c_done) / t_agq;
      if (p > best) { best = p; type = MA_GOO_AG_Q; index = iq; }
    }
    const int ir = lowest_unset(rs_done, kq);
    if (ir >= 0 && (c_done & row_mask(ir)) == row_mask(ir)) {
      const double p = 0.0;  // an output reduce-scatter makes no compute ready
      if (p > best) { best = p; type = MA_GOO_RS_Q; index = ir; }
    }
    if (type == MA_GOO_NONE && !avail) break;  // nothing left
    if (ns >= max_steps) return -set_error(MA_ERR_INVALID, "goo_plan: internal step count exceeded");
    ma_goo_step& st = steps[ns];
    std::memset(&st, 0, sizeof(st));
    if (type == MA_GOO_NONE) {
      int c = 0;
      while (!(avail >> c & 1u)) ++c;
      st.ncompute = 1;
      st.compute[0] = c;
      c_done |= 1u << c;
      ++ns;
      continue;
    }
    st.comm_type = type;
    st.comm_index = index;
    const double target = gamma * (type == MA_GOO_AG_KV ? t_agkv : type == MA_GOO_AG_Q ? t_agq : t_rsq);
    double sum = 0.0;
    for (int c = 0; c < nc && sum < target; ++c)
      if (avail >> c & 1u) {
        st.compute[st.ncompute++] = c;
        sum += t_c[c];
      }
    for (int x = 0; x < st.ncompute; ++x) c_done |= 1u << st.compute[x];
    if (type == MA_GOO_AG_KV) agkv_done |= 1u << index;
    else if (type == MA_GOO_AG_Q) agq_done |= 1u << index;
    else rs_done |= 1u << index;
    ++ns;
  }
  return ns;
}
