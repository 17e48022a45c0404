// chain.cpp -- the four calls of the path captured once as a HIP graph and
// replayed (TokenGate pages: ai.info summary "Key Contributions" item 4, the
// serving recipe captures the pruned forward pass as a graph per padded
// length).  Host code only: the capture records the kernels that the four
// calls enqueue; nothing here runs on the GPU by itself.
//
// Sizes in the graph are capacities.  The gather, the KV gather and the
// attention read the kept count from the select's n_kept at every replay
// (rows past it are padding), and with a prompt-length pointer the gate and
// the select read the prompt's length too, so one graph serves every prompt
// of its bucket.
#include <new>

#include "tg_common.hpp"

struct tg_chain {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

namespace {

// The optional KV gather forks onto `side` after the residual gather and
// joins `s` after the attention; fork/join are event edges of the capture.
tg_status run_chain(const tg_chain_desc& d, hipStream_t s, hipStream_t side, hipEvent_t fork,
                    hipEvent_t join) {
  using namespace tg;
  tg_status st = gate_score_call(d.w1_packed ? "tg_gate_score_packed" : "tg_gate_score", d.dt,
                                 d.T, d.d, d.h, d.resid, d.resid_row_stride, d.prunable,
                                 d.rms_weight, d.eps, d.w1, d.w1_packed != 0, d.b1, d.w2, d.b2,
                                 d.scores, s, d.prompt_len);
  if (st != TG_OK) return st;
  st = topk_select_call(d.T, d.scores, d.prunable, d.K, d.kept_idx, d.kept_capacity, d.n_kept,
                        d.workspace, d.workspace_bytes, s, d.prompt_len);
  if (st != TG_OK) return st;
  st = compact_gather_call(d.dt, d.T, d.N, d.d, d.resid, d.resid_row_stride, d.scores,
                           d.kept_idx, d.resid_kept, d.kept_row_stride, d.pos_kept,
                           d.score_kept, s, d.n_kept);
  if (st != TG_OK) return st;
  const bool kv = d.kv_L > 0;
  if (kv) {
    if (hipEventRecord(fork, s) != hipSuccess || hipStreamWaitEvent(side, fork, 0) != hipSuccess)
      return fail(TG_ERR_LAUNCH, "tg_chain_create: could not fork the KV gather");
    st = kv_gather_call(d.dt, d.kv_L, d.T, d.N, d.Hkv, d.D, d.kv_k_cache, d.kv_v_cache,
                        d.kept_idx, d.kv_k_kept, d.kv_v_kept, side, d.n_kept);
    if (st != TG_OK) return st;
  }
  st = bias_attn_call(d.dt, d.N, d.Hq, d.Hkv, d.D, d.q, d.k, d.v, d.attn_key_score, d.gain,
                      d.q_scale, d.softmax_scale, d.causal, d.out, d.lse, d.attn_workspace,
                      d.attn_workspace_bytes, s, d.n_kept);
  if (st != TG_OK) return st;
  if (kv && (hipEventRecord(join, side) != hipSuccess || hipStreamWaitEvent(s, join, 0) != hipSuccess))
    return fail(TG_ERR_LAUNCH, "tg_chain_create: could not join the KV gather");
  return TG_OK;
}

}  // namespace

extern "C" tg_status tg_chain_create(const tg_chain_desc* desc, tg_chain** chain) {
  using namespace tg;
  if (chain == nullptr) return fail(TG_ERR_INVALID_ARGUMENT, "tg_chain_create: chain is NULL");
  *chain = nullptr;
  if (desc == nullptr) return fail(TG_ERR_INVALID_ARGUMENT, "tg_chain_create: desc is NULL");
  hipStream_t cs = nullptr, side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  auto release = [&]() {
    if (side) (void)hipStreamDestroy(side);
    if (cs) (void)hipStreamDestroy(cs);
    if (fork) (void)hipEventDestroy(fork);
    if (join) (void)hipEventDestroy(join);
  };
  hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
  if (e == hipSuccess && desc->kv_L > 0) {
    e = hipStreamCreateWithFlags(&side, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&join, hipEventDisableTiming);
  }
  if (e != hipSuccess) {
    release();
    return fail(TG_ERR_LAUNCH, "tg_chain_create: stream/event creation failed: %s",
                hipGetErrorString(e));
  }
  e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    release();
    return fail(TG_ERR_LAUNCH, "tg_chain_create: capture failed to begin: %s",
                hipGetErrorString(e));
  }
  const tg_status st = run_chain(*desc, cs, side, fork, join);
  hipGraph_t graph = nullptr;
  e = hipStreamEndCapture(cs, &graph);
  release();
  if (st != TG_OK) {   // the failing call's message is kept
    if (graph) (void)hipGraphDestroy(graph);
    return st;
  }
  if (e != hipSuccess || graph == nullptr)
    return fail(TG_ERR_LAUNCH, "tg_chain_create: capture failed: %s", hipGetErrorString(e));
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return fail(TG_ERR_LAUNCH, "tg_chain_create: instantiation failed: %s", hipGetErrorString(e));
  }
  tg_chain* c = new (std::nothrow) tg_chain{graph, exec};
  if (c == nullptr) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(graph);
    return fail(TG_ERR_LAUNCH, "tg_chain_create: out of host memory");
  }
  *chain = c;
  clear_error();
  return TG_OK;
}

extern "C" tg_status tg_chain_launch(const tg_chain* chain, void* stream) {
  using namespace tg;
  if (chain == nullptr) return fail(TG_ERR_INVALID_ARGUMENT, "tg_chain_launch: chain is NULL");
  const hipError_t e = hipGraphLaunch(chain->exec, as_stream(stream));
  if (e != hipSuccess)
    return fail(TG_ERR_LAUNCH, "tg_chain_launch: %s", hipGetErrorString(e));
  clear_error();
  return TG_OK;
}

extern "C" void tg_chain_destroy(tg_chain* chain) {
  if (chain == nullptr) return;
  (void)hipGraphExecDestroy(chain->exec);
  (void)hipGraphDestroy(chain->graph);
  delete chain;
}
