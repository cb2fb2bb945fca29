"""Workspace reuse ordering of BatchAttention, checked on the host without a GPU.

The launches and the event calls of BatchAttention are replaced by recorders, and a small model of
in-order streams decides from the record whether each hazard is excluded:
  * before a plan writes host_ws, the previous upload (which reads host_ws on the GPU) is known to
    have completed on the host;
  * before a plan's upload overwrites int_ws, every run and merge that read it on another stream
    is known to have completed (a launch on the upload's own stream is ordered by the stream);
  * a run or merge on another stream than the upload's waits (on the GPU) for the upload;
and, with two workspaces in turn and every run merged (or settled by merge() when the merge is
fused), that the pipeline is kept: no plan's host wait reaches past the previous step's run, so the
host plans one step while the GPU still runs the one before.  Streams are torch stream objects, which compare like device streams: unequal to anything that is
not a stream, None included (`stream != None` is False)."""
import numpy as np
import pytest
import torch

import block_sparse_kv_plan_amd.attention as A


class _Ev:
    def __init__(self, *a, **k):
        self.log = None

    def record(self, stream=None):
        self.log.append(("record", self, stream))

    def synchronize(self):
        self.log.append(("sync", self))


class _Stream(torch.Stream):
    log = None

    def wait_event(self, ev):
        self.log.append(("wait", self, ev))


def _stream(i, log):
    s = _Stream(stream_id=i, device_index=0, device_type=0)
    s.log = log
    return s


class _Problem:
    tile_q = A.TILE_DECODE

    def __init__(self, fused):
        self.fused_merge = fused


def _attention(monkeypatch, fused, log, ws=0):
    """A BatchAttention whose launches append ("launch", kind, stream, workspace) to `log`."""
    monkeypatch.setattr(A.torch.cuda, "Event", _Ev)
    monkeypatch.setattr(A, "_HostOrderEvent", _Ev)
    # plan(problem, qo, kv_len, kv_indptr, host_ws[, int_ws, stream]) writes host_ws and, given
    # int_ws, uploads; upload_plan(problem, info, host_ws, int_ws, stream); run_decode and
    # merge_states (problem, info, tensors, int_ws, float_ws, stream); merge_states_upload(problem,
    # info, tensors, int_ws, float_ws, next_problem, next_info, next_host_ws, next_int_ws, stream).
    # host_ws and int_ws carry the workspace's tag.
    def plan(*a):
        log.append(("host_write", a[4]))
        if len(a) > 5 and a[5] is not None:
            log.append(("launch", "upload", a[6], a[5]))

    def merge_states_upload(*a):
        log.append(("launch", "merge", a[9], a[3]))
        log.append(("launch", "upload", a[9], a[8]))
    monkeypatch.setattr(A, "plan", plan)
    monkeypatch.setattr(A, "upload_plan", lambda *a: log.append(("launch", "upload", a[4], a[3])))
    monkeypatch.setattr(A, "run_decode", lambda *a: log.append(("launch", "run", a[-1], a[3])))
    monkeypatch.setattr(A, "merge_states", lambda *a: log.append(("launch", "merge", a[-1], a[3])))
    monkeypatch.setattr(A, "merge_states_upload", merge_states_upload)
    a = object.__new__(A.BatchAttention)
    a.problem = _Problem(fused)
    a.float_ws = None
    a.host_ws = a.int_ws = ws
    a.info = None
    a._init_order()
    for ev in (a._uploaded, a._consumed, a._merged):
        ev.log = log
    return a


def _pair(monkeypatch, fused, log):
    return [_attention(monkeypatch, fused, log, ws) for ws in (0, 1)]


def _record_of(log, ev, before):
    """(index, stream) of the last record of ev before log index `before`, or None."""
    for j in range(before - 1, -1, -1):
        e = log[j]
        if e[0] == "record" and e[1] is ev:
            return j, e[2]
    return None


def _done_on_gpu_before(log, i, stream, at):
    """Whether the launch at log index i on `stream` is complete in queue order before a command
    issued on `stream` at index `at` (same stream, or a wait on `stream` for an event recorded after
    the launch on its own stream)."""
    s_launch = log[i][2]
    if s_launch == stream:
        return True
    for j in range(i + 1, at):
        e = log[j]
        if e[0] == "wait" and e[1] == stream:
            rec = _record_of(log, e[2], j)
            if rec and rec[0] > i and _done_on_gpu_before(log, i, rec[1], rec[0]):
                return True
    return False


def _done_on_host_before(log, i, at):
    """Whether the launch at log index i is known complete on the host before index `at`: some event
    synchronized in between was recorded after it in queue order."""
    for q in range(i + 1, at):
        e = log[q]
        if e[0] == "sync":
            rec = _record_of(log, e[1], q)
            if rec and rec[0] > i and _done_on_gpu_before(log, i, rec[1], rec[0]):
                return True
    return False


def _check(log, ws=0, min_uploads=3):
    """The hazards of workspace `ws` (launches of the other workspace only share the streams)."""
    launches = [(i, e) for i, e in enumerate(log) if e[0] == "launch" and e[3] == ws]
    uploads = [i for i, e in launches if e[1] == "upload"]
    writes = [i for i, e in enumerate(log) if e[0] == "host_write" and e[1] == ws]
    assert len(uploads) >= min_uploads
    # the host writes host_ws (in the plan call, after its host waits) only once every upload
    # made from it before has completed
    for k, h in enumerate(writes):
        for u in uploads:
            if u < h:
                assert _done_on_host_before(log, u, h), f"plan {k}: previous upload not waited for"
    for k, u in enumerate(uploads):
        up_stream = log[u][2]
        for i, e in launches:
            if i >= u or e[1] == "upload":
                continue
            if e[2] != up_stream:
                assert _done_on_host_before(log, i, u), f"plan {k}: {e[1]} at {i} on another stream not waited for"
    for i, e in launches:
        if e[1] == "upload":
            continue
        last_up = max(u for u in uploads if u < i)
        assert _done_on_gpu_before(log, last_up, e[2], i), f"{e[1]} at {i} does not wait for the upload at {last_up}"


STEPS = 6
_Z = (np.zeros(2), np.zeros(1), np.zeros(2))


def _check_pipelined(log, marks):
    """marks[k] is the log length when step k began.  The host waits of plan k (k >= 1) are all for
    events recorded before the run of step k-1 was launched."""
    for k in range(1, len(marks)):
        end = marks[k + 1] if k + 1 < len(marks) else len(log)
        prev_run = next(i for i in range(marks[k - 1], marks[k]) if log[i][:2] == ("launch", "run"))
        upload = next(i for i in range(marks[k], end) if log[i][:2] == ("launch", "upload"))
        for q in range(marks[k], upload):
            if log[q][0] == "sync":
                rec = _record_of(log, log[q][1], q)
                assert rec is not None and rec[0] < prev_run, f"plan {k} waits for work queued after step {k - 1}'s run"


def _steps(pair, log, step, n=STEPS):
    marks = []
    for k in range(n):
        marks.append(len(log))
        step(pair[k % 2])
    for ws in (0, 1):
        _check(log, ws)
    return marks


@pytest.mark.parametrize("fused", [0, 1])
@pytest.mark.parametrize("copy", [False, True])
def test_run_with_merge(monkeypatch, fused, copy):
    log = []
    pair = _pair(monkeypatch, fused, log)
    s, cs = _stream(1, log), _stream(2, log)

    def step(a):
        a.plan(*_Z, stream=s, copy_stream=cs if copy else None)
        a.run(None, stream=s)
    _check_pipelined(log, _steps(pair, log, step))


@pytest.mark.parametrize("copy", [False, True])
def test_run_without_merge(monkeypatch, copy):
    """A run whose merge is never called: safe, though its plan then waits for all queued work (the
    run's event is only recorded at the next plan)."""
    log = []
    pair = _pair(monkeypatch, 0, log)
    s, cs = _stream(1, log), _stream(2, log)

    def step(a):
        a.plan(*_Z, stream=s, copy_stream=cs if copy else None)
        a.run(None, stream=s, merge=False)
    _steps(pair, log, step)


@pytest.mark.parametrize("fused", [0, 1])
@pytest.mark.parametrize("copy", [False, True])
def test_merge_on_its_own_stream(monkeypatch, fused, copy):
    log = []
    pair = _pair(monkeypatch, fused, log)
    s, cs, m = _stream(1, log), _stream(2, log), _stream(3, log)

    def step(a):
        a.plan(*_Z, stream=s, copy_stream=cs if copy else None)
        a.run(None, stream=s, merge=False)
        done = _Ev()
        done.log = log
        done.record(s)
        m.wait_event(done)
        a.merge(None, stream=m)
    _check_pipelined(log, _steps(pair, log, step))


def test_replan_without_run(monkeypatch):
    """Two plans in a row with no run between them: the second waits for the first upload."""
    log = []
    a = _attention(monkeypatch, 0, log)
    s = _stream(1, log)
    for _ in range(3):
        a.plan(*_Z, stream=s)
    a.run(None, stream=s)
    _check(log)


def test_checker_catches_a_missing_run_wait(monkeypatch):
    """The model is not vacuous: dropping the host wait for the last run on another stream than
    the upload's (what a `stream != None` test once did in fused mode) fails the check."""
    log = []
    pair = _pair(monkeypatch, 1, log)
    s, cs = _stream(1, log), _stream(2, log)
    assert (s != None) is False  # noqa: E711 -- the trap this file guards against
    for a in pair:
        a._consumed.synchronize = lambda: None

    def step(a):
        a.plan(*_Z, stream=s, copy_stream=cs)
        a.run(None, stream=s)
    with pytest.raises(AssertionError, match="not waited for"):
        _steps(pair, log, step)


def test_checker_catches_lockstep(monkeypatch):
    """...and a plan that waits for an upload event recorded only at that plan (behind the other
    workspace's run) fails the pipelining check."""
    log = []
    pair = _pair(monkeypatch, 1, log)
    s = _stream(1, log)
    for a in pair:
        a._recorded = lambda ev: None

    def step(a):
        a.plan(*_Z, stream=s)
        a.run(None, stream=s)
    marks = _steps(pair, log, step)
    with pytest.raises(AssertionError, match="waits for work queued after"):
        _check_pipelined(log, marks)


@pytest.mark.parametrize("fused", [0, 1])
def test_deferred_uploads_ride_on_the_other_workspace_merge(monkeypatch, fused):
    """Two workspaces in turn, in one stream: each plan's upload is deferred and made in the same
    launch as the other workspace's merge of the previous step (upload() for the first step, a
    plain merge after the last).  Every hazard is excluded and the pipeline is kept."""
    log = []
    pair = _pair(monkeypatch, fused, log)
    s = _stream(1, log)
    marks, prev = [], None
    for k in range(STEPS):
        a = pair[k % 2]
        marks.append(len(log))
        a.plan(*_Z, stream=s, defer_upload=True)
        with pytest.raises(RuntimeError, match="deferred"):
            a.run(None, stream=s)
        if prev is None:
            a.upload(s)
        else:
            prev.merge(None, stream=s, upload_next=a)
        a.run(None, stream=s, merge=False)
        prev = a
    prev.merge(None, stream=s)
    for ws in (0, 1):
        _check(log, ws)
    _check_pipelined(log, marks)


def test_deferred_upload_stream_and_target_checks(monkeypatch):
    log = []
    a, b = _pair(monkeypatch, 0, log)
    s, cs = _stream(1, log), _stream(2, log)
    with pytest.raises(RuntimeError, match="no deferred upload"):
        a.upload(s)
    a.plan(*_Z, stream=s, copy_stream=cs, defer_upload=True)
    with pytest.raises(ValueError, match="stream its plan named"):
        a.upload(s)
    b.plan(*_Z, stream=s)
    b.run(None, stream=s, merge=False)
    with pytest.raises(ValueError, match="stream its plan named"):
        b.merge(None, stream=s, upload_next=a)
    with pytest.raises(ValueError, match="another workspace"):
        b.merge(None, stream=s, upload_next=b)
    a.upload(cs)
    b.merge(None, stream=s)
    a.run(None, stream=s)
    # a later plan supersedes a deferred upload that was never made
    a.plan(*_Z, stream=s, defer_upload=True)
    a.plan(*_Z, stream=s)
    a.run(None, stream=s)
    for ws in (0, 1):
        _check(log, ws, min_uploads=1)
