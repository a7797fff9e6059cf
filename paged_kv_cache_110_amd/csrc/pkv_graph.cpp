// Graph-captured decode step with batch buckets (devpress "nano-vllm解读",
// "CUDAGraph优化"; AIInfraGuide 3.6, section 5): one HIP graph per batch
// bucket, each holding every layer's store and decode over static buffers
// sized for the largest bucket.  A step of `batch` rows pads the rows up to
// its bucket (slot -1, context length 0) and replays that bucket's graph, so
// the host issues two launches per step instead of three per layer.
#include <algorithm>
#include <new>
#include <vector>

#include "pkv.h"
#include "pkv_internal.h"

struct pkv_decode_graph {
  pkv_decode_step step;  // per-layer pointer arrays re-pointed at the copies below
  std::vector<const void*> q, key, value;
  std::vector<void*> k_cache, v_cache, out;
  std::vector<int32_t> buckets;
  std::vector<hipGraph_t> graphs;
  std::vector<hipGraphExec_t> execs;

  ~pkv_decode_graph() {
    for (hipGraphExec_t e : execs) (void)hipGraphExecDestroy(e);
    for (hipGraph_t g : graphs) (void)hipGraphDestroy(g);
  }
};

namespace {

constexpr int32_t kMaxGraphBatch = 512;  // larger batches run eagerly

std::vector<int32_t> bucket_list(int32_t max_batch) {
  std::vector<int32_t> b;
  for (int32_t x : {1, 2, 4, 8})
    if (x <= max_batch) b.push_back(x);
  for (int32_t x = 16; x <= max_batch; x += 16) b.push_back(x);
  if (b.back() != max_batch) b.push_back(max_batch);
  return b;
}

bool step_pointers_ok(const pkv_decode_step* s) {
  if (!s || s->layers < 1 || s->max_batch < 1 || s->max_batch > kMaxGraphBatch) return false;
  if (!s->slot_mapping || !s->context_lens || !s->block_tables || !s->workspace) return false;
  if (!s->q || !s->key || !s->value || !s->k_cache || !s->v_cache || !s->out) return false;
  return true;
}

// Every layer's store and decode over rows [0, batch) (batch >= 1), as one
// fused launch per layer (pkv_store_decode: the new token goes to position
// context_lens[b] - 1 through the block table, the slot_mapping entry the
// pages' metadata gives it); each call runs its own argument checks.
pkv_status enqueue_step(const pkv_decode_step& s, int32_t batch, hipStream_t stream) {
  for (int32_t l = 0; l < s.layers; ++l) {
    const pkv_status st = pkv_store_decode(
        s.out[l], s.q[l], s.key[l], s.key_stride, s.value[l], s.value_stride, s.k_cache[l],
        s.v_cache[l], s.block_tables, s.context_lens, batch, s.H_q, s.H_kv, s.d, s.num_blocks,
        s.block_size, s.max_blocks_per_seq, s.softmax_scale, s.workspace, s.workspace_bytes,
        stream);
    if (st != PKV_OK) return st;
  }
  return PKV_OK;
}

// Captures the step at `batch` rows on `stream` and instantiates it.
pkv_status capture(const pkv_decode_step& s, int32_t batch, hipStream_t stream,
                   hipGraph_t* graph, hipGraphExec_t* exec) {
  *graph = nullptr;
  *exec = nullptr;
  if (hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal) != hipSuccess)
    return PKV_ELAUNCH;
  const pkv_status st = enqueue_step(s, batch, stream);
  const hipError_t end = hipStreamEndCapture(stream, graph);  // always leave capture mode
  if (st != PKV_OK) return st;
  if (end != hipSuccess || !*graph) return PKV_ELAUNCH;
  if (hipGraphInstantiateWithFlags(exec, *graph, 0) != hipSuccess) return PKV_ELAUNCH;
  return PKV_OK;
}

}  // namespace

extern "C" {

int32_t pkv_decode_graph_bucket(int32_t max_batch, int32_t batch) {
  if (max_batch < 1 || max_batch > kMaxGraphBatch || batch < 1 || batch > max_batch) return -1;
  const std::vector<int32_t> b = bucket_list(max_batch);
  return *std::lower_bound(b.begin(), b.end(), batch);
}

pkv_status pkv_decode_step_run(const pkv_decode_step* step, int32_t batch, hipStream_t stream) {
  if (!step_pointers_ok(step) || batch < 0 || batch > step->max_batch) return PKV_EINVAL;
  if (batch == 0) return PKV_OK;
  return enqueue_step(*step, batch, stream);
}

pkv_status pkv_decode_graph_create(const pkv_decode_step* step, pkv_decode_graph** graph) {
  if (!graph) return PKV_EINVAL;
  *graph = nullptr;
  if (!step_pointers_ok(step)) return PKV_EINVAL;
  const size_t need = pkv_decode_workspace_size(step->max_batch, step->H_q, step->H_kv, step->d,
                                                step->block_size, step->max_blocks_per_seq);
  if (need == 0 || step->workspace_bytes < need) return PKV_EINVAL;

  pkv_decode_graph* g = new (std::nothrow) pkv_decode_graph();
  if (!g) return PKV_ELAUNCH;
  const size_t L = (size_t)step->layers;
  g->step = *step;
  g->q.assign(step->q, step->q + L);
  g->key.assign(step->key, step->key + L);
  g->value.assign(step->value, step->value + L);
  g->k_cache.assign(step->k_cache, step->k_cache + L);
  g->v_cache.assign(step->v_cache, step->v_cache + L);
  g->out.assign(step->out, step->out + L);
  g->step.q = g->q.data();
  g->step.key = g->key.data();
  g->step.value = g->value.data();
  g->step.k_cache = g->k_cache.data();
  g->step.v_cache = g->v_cache.data();
  g->step.out = g->out.data();
  g->buckets = bucket_list(step->max_batch);

  // The set-up below runs on a stream of its own, so first let every write the
  // caller has enqueued to the static buffers and the workspace (fills, copies
  // on any stream) finish.
  if (hipDeviceSynchronize() != hipSuccess) {
    delete g;
    return PKV_ELAUNCH;
  }
  hipStream_t s = nullptr;
  if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) {
    delete g;
    return PKV_ELAUNCH;
  }
  // all rows padding, then one eager step: checks every argument, loads the
  // kernels and leaves the workspace's share counter at zero
  pkv_status st = pkv::launch_pad_batch(step->slot_mapping, step->context_lens, 0,
                                        step->max_batch, s) == hipSuccess
                      ? enqueue_step(g->step, step->max_batch, s)
                      : PKV_ELAUNCH;
  if (st == PKV_OK && hipStreamSynchronize(s) != hipSuccess) st = PKV_ELAUNCH;
  for (size_t i = 0; st == PKV_OK && i < g->buckets.size(); ++i) {
    hipGraph_t gr;
    hipGraphExec_t ex;
    st = capture(g->step, g->buckets[i], s, &gr, &ex);
    if (gr) g->graphs.push_back(gr);
    if (ex) g->execs.push_back(ex);
  }
  if (hipStreamSynchronize(s) != hipSuccess && st == PKV_OK) st = PKV_ELAUNCH;
  (void)hipStreamDestroy(s);
  if (st != PKV_OK) {
    delete g;
    return st;
  }
  *graph = g;
  return PKV_OK;
}

pkv_status pkv_decode_graph_replay(pkv_decode_graph* graph, int32_t batch, hipStream_t stream) {
  if (!graph || batch < 0 || batch > graph->step.max_batch) return PKV_EINVAL;
  if (batch == 0) return PKV_OK;
  const auto it = std::lower_bound(graph->buckets.begin(), graph->buckets.end(), batch);
  const size_t i = (size_t)(it - graph->buckets.begin());
  if (pkv::launch_pad_batch(graph->step.slot_mapping, graph->step.context_lens, batch, *it,
                            stream) != hipSuccess)
    return PKV_ELAUNCH;
  return hipGraphLaunch(graph->execs[i], stream) == hipSuccess ? PKV_OK : PKV_ELAUNCH;
}

void pkv_decode_graph_destroy(pkv_decode_graph* graph) {
  if (!graph) return;
  (void)hipDeviceSynchronize();  // no replay may still be running
  delete graph;
}

}  // extern "C"
