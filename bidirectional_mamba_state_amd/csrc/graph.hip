// Decode loop of one active block as a HIP graph (the C ABI's bdssm_decode_graph_*): the
// block's denoising steps and its commit are recorded once by stream capture and replayed
// with one launch. Host code only.
#include <new>

#include "bdssm.h"
#include "internal.h"

struct bdssm_decode_graph {
    hipGraph_t graph;
    hipGraphExec_t exec;
};

extern "C" bdssm_status bdssm_decode_graph_create(const bdssm_dims *dims, int32_t block_len, int32_t steps,
                                                  float *h, void *h_ops, const bdssm_seq *fwd, const bdssm_seq *rev,
                                                  const float *A, const float *D, void *const *y,
                                                  const bdssm_seq *clean, void *y_commit, void *stream,
                                                  bdssm_decode_graph **out)
{
    if (out)
        *out = nullptr;
    if (!dims || !out || !stream)
        return BDSSM_ERR_NULL;
    if (steps < 0)
        return BDSSM_ERR_SHAPE;
    if (steps > 0 && (!fwd || !rev || !y))
        return BDSSM_ERR_NULL;
    if (steps == 0 && !clean)
        return BDSSM_ERR_NULL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal) != hipSuccess) {
        (void)hipGetLastError();
        return BDSSM_ERR_HIP;
    }
    // record the calls; on the first failure end the capture and drop what was recorded
    bdssm_status rc = BDSSM_OK;
    for (int32_t k = 0; k < steps && rc == BDSSM_OK; ++k)
        rc = h_ops ? bdssm_block_step_ops(dims, block_len, h_ops, &fwd[k], &rev[k], A, D, A, nullptr, y[k], stream)
                   : bdssm_block_step(dims, block_len, h, &fwd[k], &rev[k], A, D, y[k], stream);
    if (rc == BDSSM_OK && clean) {
        // the next block's steps read the advanced state: with h_ops, the commit refreshes it
        rc = h_ops ? bdssm_commit_refresh(dims, block_len, clean, A, D, h, h_ops, BDSSM_STATE_OPS, y_commit, stream)
                   : bdssm_commit(dims, block_len, clean, A, D, h, y_commit, stream);
    }
    hipGraph_t graph = nullptr;
    const hipError_t ce = hipStreamEndCapture(st, &graph);
    if (rc != BDSSM_OK || ce != hipSuccess) {
        if (graph)
            (void)hipGraphDestroy(graph);
        (void)hipGetLastError();
        return rc != BDSSM_OK ? rc : BDSSM_ERR_HIP;
    }
    hipGraphExec_t exec = nullptr;
    if (hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess) {
        (void)hipGraphDestroy(graph);
        (void)hipGetLastError();
        return BDSSM_ERR_HIP;
    }
    bdssm_decode_graph *g = new (std::nothrow) bdssm_decode_graph{graph, exec};
    if (!g) {
        (void)hipGraphExecDestroy(exec);
        (void)hipGraphDestroy(graph);
        return BDSSM_ERR_HIP;
    }
    *out = g;
    return BDSSM_OK;
}

extern "C" bdssm_status bdssm_decode_graph_launch(const bdssm_decode_graph *graph, void *stream)
{
    if (!graph)
        return BDSSM_ERR_NULL;
    if (hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream)) != hipSuccess) {
        (void)hipGetLastError();
        return BDSSM_ERR_HIP;
    }
    return BDSSM_OK;
}

extern "C" void bdssm_decode_graph_destroy(bdssm_decode_graph *graph)
{
    if (!graph)
        return;
    (void)hipGraphExecDestroy(graph->exec);
    (void)hipGraphDestroy(graph->graph);
    delete graph;
}
