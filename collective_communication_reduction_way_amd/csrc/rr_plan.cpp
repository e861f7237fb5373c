// rr_plan.cpp -- the ring / hierarchical chunk scheduler and byte accounting
// (host only; no GPU needed, so the CPU tests exercise it through the C ABI).
//
// Ring: page "LLM Parallelism 基础", section "Ring AllReduce".  The data of
// every rank is cut evenly into p chunks and the ranks form a logical ring in
// which each rank talks only to its successor.  Phase one (reduce-scatter)
// has p-1 steps; in each step a rank passes one chunk to its successor, which
// adds the chunk into its own copy.  Phase two (all-gather) has p-1 steps in
// which the successor overwrites its copy instead.  The schedule below is
// built from the forwarding rule rather than from a closed formula: in
// reduce-scatter step 0 rank r sends its predecessor's chunk (r-1), and in
// every later step it forwards the chunk it received in the step before; in
// all-gather step 0 rank r sends the chunk it owns (r) and then again forwards
// what it received.  That rule leaves rank c holding the complete chunk c after
// phase one, as the page states.
//
// Byte accounting: page "分布式训练/推理", section "Ring all-reduce 的带宽账":
// in each phase every device sends (N-1)/N of the full tensor.  Hierarchical
// traffic: page "大模型并行的最小闭环：集合通信、TP、FSDP/ZeRO-3 到权重分片",
// section "Source Log: 2026-05-05" (对比数据量): without the hierarchy each
// member ships its own B bytes across nodes (G*B per node); with it only the
// representative ships B.
#include "rr_plan.h"

#include <string.h>

namespace rr {

std::vector<Transfer> ring_schedule(int p) {
  std::vector<Transfer> out;
  if (p < 2) return out;
  out.reserve(static_cast<size_t>(2 * (p - 1) * p));
  for (int phase = 0; phase < 2; ++phase) {
    // what each rank sends in the current step
    std::vector<int> sending(p);
    for (int r = 0; r < p; ++r) sending[r] = phase == 0 ? (r + p - 1) % p : r;
    for (int s = 0; s < p - 1; ++s) {
      std::vector<int> received(p);
      for (int r = 0; r < p; ++r) {
        const int dst = (r + 1) % p;
        out.push_back(Transfer{phase, s, r, dst, sending[r]});
        received[dst] = sending[r];
      }
      sending = received;  // forward what just arrived
    }
  }
  return out;
}

void chunk_bounds(int p, uint64_t n, uint64_t* bounds) {
  // c*n fits in 64 bits: the API limits n to 2^56 and p to 64.
  for (int c = 0; c <= p; ++c) bounds[c] = (static_cast<uint64_t>(c) * n) / static_cast<uint64_t>(p);
}

size_t elem_size(rr_dtype_t dt) {
  switch (dt) {
    case RR_INT32: return 4;
    case RR_FLOAT32: return 4;
    case RR_BFLOAT16: return 2;
    case RR_FLOAT16: return 2;
  }
  return 0;
}

}  // namespace rr

extern "C" {

int rr_ring_schedule(int p, int* phase, int* step, int* src, int* dst, int* chunk, int cap) {
  if (p < 1 || p > RR_MAX_RANKS) return -1;
  const std::vector<rr::Transfer> t = rr::ring_schedule(p);
  const int total = static_cast<int>(t.size());
  const int m = cap < total ? cap : total;
  for (int i = 0; i < m; ++i) {
    if (phase) phase[i] = t[i].phase;
    if (step) step[i] = t[i].step;
    if (src) src[i] = t[i].src;
    if (dst) dst[i] = t[i].dst;
    if (chunk) chunk[i] = t[i].chunk;
  }
  return total;
}

rr_status_t rr_chunk_bounds(int p, size_t n, size_t* bounds) {
  if (p < 1 || p > RR_MAX_RANKS || !bounds || n > (1ull << 56)) return RR_ERROR_INVALID_ARGUMENT;
  uint64_t b[RR_MAX_RANKS + 1];
  rr::chunk_bounds(p, n, b);
  for (int c = 0; c <= p; ++c) bounds[c] = static_cast<size_t>(b[c]);
  return RR_SUCCESS;
}

rr_status_t rr_algorithmic_bytes(rr_coll_t coll, int p, size_t n, rr_dtype_t dtype, int in_place,
                                 uint64_t* bytes) {
  const uint64_t s = rr::elem_size(dtype);
  if (!bytes || s == 0 || p < 1 || p > RR_MAX_RANKS || n > (1ull << 56)) return RR_ERROR_INVALID_ARGUMENT;
  const uint64_t P = static_cast<uint64_t>(p);
  const uint64_t ns = static_cast<uint64_t>(n) * s;
  switch (coll) {
    case RR_COLL_ALL_REDUCE: *bytes = 2 * P * ns; return RR_SUCCESS;
    case RR_COLL_REDUCE_SCATTER:
    case RR_COLL_ALL_GATHER:
    case RR_COLL_REDUCE: *bytes = (P + 1) * ns; return RR_SUCCESS;
    case RR_COLL_BROADCAST: *bytes = ns + (in_place ? (P - 1) : P) * ns; return RR_SUCCESS;
    case RR_COLL_SCATTER:
    case RR_COLL_GATHER:
      if (n % P) return RR_ERROR_INVALID_ARGUMENT;
      *bytes = in_place ? 2 * (ns / P) * (P - 1) : 2 * ns;
      return RR_SUCCESS;
  }
  return RR_ERROR_INVALID_ARGUMENT;
}

rr_status_t rr_ring_bytes_per_rank(int p, size_t n, rr_dtype_t dtype, uint64_t* sent_rs, uint64_t* sent_ag) {
  const uint64_t s = rr::elem_size(dtype);
  if (!sent_rs || !sent_ag || s == 0 || p < 1 || p > RR_MAX_RANKS || n > (1ull << 56))
    return RR_ERROR_INVALID_ARGUMENT;
  uint64_t b[RR_MAX_RANKS + 1];
  rr::chunk_bounds(p, n, b);
  uint64_t per[2][RR_MAX_RANKS];
  memset(per, 0, sizeof(per));
  for (const rr::Transfer& t : rr::ring_schedule(p)) per[t.phase][t.src] += (b[t.chunk + 1] - b[t.chunk]) * s;
  uint64_t mx[2] = {0, 0};
  for (int ph = 0; ph < 2; ++ph)
    for (int r = 0; r < p; ++r) mx[ph] = per[ph][r] > mx[ph] ? per[ph][r] : mx[ph];
  *sent_rs = mx[0];
  *sent_ag = mx[1];
  return RR_SUCCESS;
}

rr_status_t rr_hier_traffic(int p, int group_size, uint64_t bytes_per_rank, uint64_t* intra_per_group,
                            uint64_t* cross_per_group_flat, uint64_t* cross_per_group_hier) {
  if (p < 1 || p > RR_MAX_RANKS || group_size < 1 || p % group_size || !intra_per_group ||
      !cross_per_group_flat || !cross_per_group_hier)
    return RR_ERROR_INVALID_ARGUMENT;
  const uint64_t G = static_cast<uint64_t>(group_size);
  *intra_per_group = G * bytes_per_rank;
  *cross_per_group_flat = G * bytes_per_rank;
  *cross_per_group_hier = bytes_per_rank;
  return RR_SUCCESS;
}

// Alpha-beta cost model.  Page "分布式训练/推理": a message costs
// alpha + bytes/bandwidth (section "从单卡到多卡"); the ring all-reduce runs
// 2(N-1) rounds of S/N bytes per device (section "Ring all-reduce 的带宽账").
// Page "大模型并行的最小闭环：集合通信、TP、FSDP/ZeRO-3 到权重分片", section
// "总体时间模型": flat T_slow(B*N) against hierarchical T_fast(B*N) + T_slow(B).
namespace {

bool link_ok(const rr_link_t& l) { return l.alpha_s >= 0.0 && l.bytes_per_s > 0.0; }

double message_time(const rr_link_t& l, double bytes) { return l.alpha_s + bytes / l.bytes_per_s; }

}  // namespace

rr_status_t rr_cost_ring_all_reduce(int p, double bytes, rr_link_t link, double* seconds) {
  if (p < 1 || p > RR_MAX_RANKS || !(bytes >= 0.0) || !link_ok(link) || !seconds) return RR_ERROR_INVALID_ARGUMENT;
  const double rounds = 2.0 * (p - 1);
  *seconds = rounds * message_time(link, bytes / p);
  return RR_SUCCESS;
}

rr_status_t rr_cost_hier_all_reduce(int group_size, double bytes, rr_link_t fast, rr_link_t slow, double* t_flat,
                                    double* t_hier, int* use_hier) {
  if (group_size < 1 || group_size > RR_MAX_RANKS || !(bytes >= 0.0) || !link_ok(fast) || !link_ok(slow))
    return RR_ERROR_INVALID_ARGUMENT;
  const double node_bytes = static_cast<double>(group_size) * bytes;
  const double flat = message_time(slow, node_bytes);
  const double hier = message_time(fast, node_bytes) + message_time(slow, bytes);
  if (t_flat) *t_flat = flat;
  if (t_hier) *t_hier = hier;
  if (use_hier) *use_hier = hier < flat ? 1 : 0;
  return RR_SUCCESS;
}

}  // extern "C"
