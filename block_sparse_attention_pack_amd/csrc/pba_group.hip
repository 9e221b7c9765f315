// Group preference objectives and their first-order surrogate coefficients
// ("GroupDPO" page, section "core formulas").  For a batch of groups, each
// with non-empty disjoint positive and negative response sets, and the
// per-response log-prob sums of the policy and of the frozen reference:
//
//   u_i     = beta (pol_i / len_i - ref_i / len_i)
//   L_group = (1/|G|) sum_g phi_g(u[P_g], u[N_g])
//   c_i     = (1/|G|) sum_{g containing i} d phi_g / d u_i
//   w_i     = alpha sum_{g: i in P_g} 1 / (|G| |P_g|)   (positive-NLL weight)
//   nll     = alpha (1/|G|) sum_g mean_{i in P_g} (-pol_i / len_i)
//
// with phi one of four group forms, each the DPO loss -log sigmoid(u+ - u-)
// for a single pair: all-pairs (mean pair loss), margin (pair loss of the
// mean rewards), MPO (log-sum-exp of all minus log-sum-exp of the
// positives) and softmax (mean over positives of the log-softmax loss
// against all negatives).
//
// The work is a few scalars per response, so one workgroup does all of it,
// in fp64, with every sum in a fixed order (deterministic):
//   1. each entry's reward u into LDS; each group checked (thread per group)
//   2. thread per group: phi_g and d phi_g / d u of its entries into LDS
//   3. thread per entry: the first entry of each response sums the terms of
//      all its entries in entry order and writes c_i and w_i; responses in no
//      group get 0
#include "pba_next.h"

namespace pba {
namespace {

constexpr int kGThreads = 256;

__device__ __forceinline__ double sigmoid_d(double x) {
  if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
  const double e = exp(x);
  return e / (1.0 + e);
}

__device__ __forceinline__ double neg_log_sigmoid_d(double x) {
  return x >= 0.0 ? log1p(exp(-x)) : log1p(exp(x)) - x;
}

__global__ void __launch_bounds__(kGThreads) group_coef(GroupArgs a) {
  __shared__ double u_e[kMaxGroupEntries];   // reward of each entry's response
  __shared__ double g_e[kMaxGroupEntries];   // (1/|G|) d phi_g / d u of each entry
  __shared__ float w_e[kMaxGroupEntries];    // positive-NLL weight of each entry
  __shared__ int m_e[kMaxGroupEntries];      // response of each entry
  __shared__ double phi_g[kMaxGroups];
  __shared__ double nll_g[kMaxGroups];
  __shared__ int first_bad;                  // group * 16 + code, minimum over groups

  const int tid = threadIdx.x;
  const int G = a.n_groups, E = a.n_entries;
  if (tid == 0) first_bad = 0x7fffffff;
  for (int e = tid; e < E; e += kGThreads) {
    const int i = a.member[e];
    m_e[e] = i;
    const bool ok = i >= 0 && i < a.n_resp && a.resp_len[i] > 0;
    const double len = ok ? (double)a.resp_len[i] : 1.0;
    u_e[e] = ok ? a.beta * ((double)a.pol[i] / len - (double)a.ref[i] / len) : 0.0;
  }
  __syncthreads();

  // 1. validation; the smallest offending group wins, with its first failing
  //    check (the checks run in a fixed order)
  for (int g = tid; g < G; g += kGThreads) {
    const int lo = a.group_ptr[g], hi = a.group_ptr[g + 1];
    int code = 0;
    if (lo < 0 || hi < lo || hi > E || (g == 0 && lo != 0) || (g == G - 1 && hi != E)) {
      code = kGroupPtr;
    } else {
      int np = 0, nn = 0;
      for (int e = lo; e < hi && !code; ++e) {
        const int i = m_e[e];
        if (i < 0 || i >= a.n_resp) code = kGroupMember;
        else if (a.resp_len[i] <= 0) code = kGroupLength;
        for (int f = lo; f < e && !code; ++f)
          if (m_e[f] == i) code = kGroupDuplicate;
        (a.positive[e] ? np : nn) += 1;
      }
      if (!code && (np == 0 || nn == 0)) code = kGroupEmpty;
    }
    if (code) atomicMin(&first_bad, g * 16 + code);
  }
  __syncthreads();
  if (first_bad != 0x7fffffff) {
    if (tid == 0) {
      a.status[0] = first_bad & 15;
      a.status[1] = first_bad >> 4;
      if (a.loss) a.loss[0] = a.loss[1] = __builtin_nanf("");
    }
    for (int i = tid; i < a.n_resp; i += kGThreads) {
      a.coef[i] = __builtin_nanf("");
      if (a.nll_w) a.nll_w[i] = __builtin_nanf("");
    }
    return;
  }
  if (tid == 0) a.status[0] = a.status[1] = 0;

  // 2. one group per thread
  const double invG = 1.0 / G;
  for (int g = tid; g < G; g += kGThreads) {
    const int lo = a.group_ptr[g], hi = a.group_ptr[g + 1];
    int np = 0, nn = 0;
    double sum_pos_nll = 0.0, mean_p = 0.0, mean_n = 0.0, max_all = -__builtin_inf(), max_p = -__builtin_inf();
    for (int e = lo; e < hi; ++e) {
      const double u = u_e[e];
      g_e[e] = 0.0;
      max_all = fmax(max_all, u);
      if (a.positive[e]) {
        ++np;
        mean_p += u;
        max_p = fmax(max_p, u);
        const int i = m_e[e];
        sum_pos_nll -= (double)a.pol[i] / (double)a.resp_len[i];
      } else {
        ++nn;
        mean_n += u;
      }
    }
    mean_p /= np;
    mean_n /= nn;
    for (int e = lo; e < hi; ++e) w_e[e] = a.positive[e] ? (float)(a.alpha * invG / np) : 0.f;
    nll_g[g] = sum_pos_nll / np;
    double phi = 0.0;
    switch (a.objective) {
      case kObjAllPairs: {
        const double wpair = 1.0 / ((double)np * nn);
        for (int e = lo; e < hi; ++e) {
          if (!a.positive[e]) continue;
          for (int f = lo; f < hi; ++f) {
            if (a.positive[f]) continue;
            const double x = u_e[e] - u_e[f];
            const double s = sigmoid_d(-x) * wpair;
            g_e[e] -= s;
            g_e[f] += s;
            phi += neg_log_sigmoid_d(x) * wpair;
          }
        }
        break;
      }
      case kObjMargin: {
        const double x = mean_p - mean_n;
        const double s = sigmoid_d(-x);
        for (int e = lo; e < hi; ++e) g_e[e] = a.positive[e] ? -s / np : s / nn;
        phi = neg_log_sigmoid_d(x);
        break;
      }
      case kObjMpo: {
        double s_all = 0.0, s_p = 0.0;
        for (int e = lo; e < hi; ++e) {
          s_all += exp(u_e[e] - max_all);
          if (a.positive[e]) s_p += exp(u_e[e] - max_p);
        }
        const double lse_all = max_all + log(s_all), lse_p = max_p + log(s_p);
        for (int e = lo; e < hi; ++e) {
          const double pa = exp(u_e[e] - lse_all);
          g_e[e] = a.positive[e] ? pa - exp(u_e[e] - lse_p) : pa;
        }
        phi = lse_all - lse_p;
        break;
      }
      default: {  // kObjSoftmax
        double max_n = -__builtin_inf();
        for (int e = lo; e < hi; ++e)
          if (!a.positive[e]) max_n = fmax(max_n, u_e[e]);
        for (int e = lo; e < hi; ++e) {
          if (!a.positive[e]) continue;
          const double ui = u_e[e], z = fmax(ui, max_n);
          double s = exp(ui - z);
          for (int f = lo; f < hi; ++f)
            if (!a.positive[f]) s += exp(u_e[f] - z);
          const double lse = z + log(s);
          g_e[e] += (exp(ui - lse) - 1.0) / np;
          for (int f = lo; f < hi; ++f)
            if (!a.positive[f]) g_e[f] += exp(u_e[f] - lse) / np;
          phi += (lse - ui) / np;
        }
        break;
      }
    }
    for (int e = lo; e < hi; ++e) g_e[e] *= invG;
    phi_g[g] = phi;
  }
  for (int i = tid; i < a.n_resp; i += kGThreads) {
    a.coef[i] = 0.f;
    if (a.nll_w) a.nll_w[i] = 0.f;
  }
  __syncthreads();  // also orders the zero fill above before the writes below

  // 3. per response, over its entries in entry order (the first entry owns it)
  for (int e = tid; e < E; e += kGThreads) {
    const int i = m_e[e];
    bool owner = true;
    for (int f = 0; f < e && owner; ++f) owner = m_e[f] != i;
    if (!owner) continue;
    double c = 0.0, w = 0.0;
    for (int f = e; f < E; ++f) {
      if (m_e[f] != i) continue;
      c += g_e[f];
      w += w_e[f];
    }
    a.coef[i] = (float)c;
    if (a.nll_w) a.nll_w[i] = (float)w;
  }
  if (tid == 0 && a.loss) {
    double l = 0.0, n = 0.0;
    for (int g = 0; g < G; ++g) {
      l += phi_g[g];
      n += nll_g[g];
    }
    a.loss[0] = (float)(l * invG);
    a.loss[1] = (float)(a.alpha * n * invG);
  }
}

}  // namespace

hipError_t launch_group_coef(const GroupArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(group_coef, dim3(1), dim3(kGThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pba
