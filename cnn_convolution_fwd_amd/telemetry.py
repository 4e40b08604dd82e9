"""Shader clock and board power of the GPU while a benchmark runs.

Matrix-core throughput on this board is bounded by its power limit: under a
sustained MFMA load the shader clock drops well below its 2.4 GHz peak, so a
throughput figure means little without the clock and power it was taken at.
A background thread samples both while the caller's launches run and reports
median / min / max.

Sources, tried in order: the amdsmi Python bindings shipped with ROCm
(``/opt/rocm/share/amd_smi``), then the card's hwmon files in sysfs
(``freq1_input`` in Hz for the shader clock, ``power1_average`` or
``power1_input`` in microwatts).  The device is matched by its PCI address,
read from the HIP runtime.  When neither source answers, the summary says so
and holds no numbers.
"""
from __future__ import annotations

import ctypes
import glob
import os
import statistics
import sys
import threading
import time
from typing import Callable, Dict, List, Optional


def pci_bus_id(device: int = 0) -> Optional[str]:
    """'dddd:bb:dd.f' of HIP device ``device`` (lower case), or None."""
    for name in ("libamdhip64.so", "libamdhip64.so.7", "libamdhip64.so.6"):
        try:
            lib = ctypes.CDLL(name)
            break
        except OSError:
            lib = None
    if lib is None:
        return None
    buf = ctypes.create_string_buffer(64)
    try:
        if lib.hipDeviceGetPCIBusId(buf, 64, device) != 0:
            return None
    except AttributeError:
        return None
    return buf.value.decode().lower() or None


def _sysfs_reader(bdf: Optional[str]) -> Optional[Callable[[], Dict[str, float]]]:
    dirs = []
    if bdf:
        dirs = glob.glob("/sys/bus/pci/devices/%s/hwmon/hwmon*" % bdf)
    if not dirs:
        return None
    d = dirs[0]
    freq = os.path.join(d, "freq1_input")
    pw = next((os.path.join(d, f) for f in ("power1_average", "power1_input") if os.path.exists(os.path.join(d, f))),
              None)
    if not os.path.exists(freq) and pw is None:
        return None

    def read() -> Dict[str, float]:
        out = {}
        try:
            with open(freq) as f:
                out["sclk_mhz"] = int(f.read()) / 1e6
        except (OSError, ValueError):
            pass
        if pw:
            try:
                with open(pw) as f:
                    out["power_w"] = int(f.read()) / 1e6
            except (OSError, ValueError):
                pass
        return out

    return read


def _num(v) -> Optional[float]:
    if isinstance(v, dict):
        v = v.get("value", None)
    try:
        f = float(v)
    except (TypeError, ValueError):
        return None
    return f if f == f and 0 < f < 65535 else None


def _amdsmi_reader(bdf: Optional[str]) -> Optional[Callable[[], Dict[str, float]]]:
    path = "/opt/rocm/share/amd_smi"
    if os.path.isdir(path) and path not in sys.path:
        sys.path.append(path)
    try:
        import amdsmi  # type: ignore
        amdsmi.amdsmi_init()
        handles = amdsmi.amdsmi_get_processor_handles()
    except Exception:
        return None
    h = None
    for cand in handles:
        try:
            if bdf and amdsmi.amdsmi_get_gpu_device_bdf(cand).lower() == bdf:
                h = cand
                break
        except Exception:
            continue
    if h is None:
        if len(handles) != 1:
            return None
        h = handles[0]

    def read() -> Dict[str, float]:
        out = {}
        try:
            m = amdsmi.amdsmi_get_gpu_metrics_info(h)
            act = m.get("average_gfx_activity")
            if isinstance(act, (int, float)) and 0 <= act <= 100:
                out["activity_pct"] = float(act)
            for key in ("current_gfxclk", "average_gfxclk_frequency"):
                v = _num(m.get(key))
                if v:
                    out["sclk_mhz"] = v
                    break
            for key in ("current_socket_power", "average_socket_power"):
                v = _num(m.get(key))
                if v:
                    out["power_w"] = v
                    break
        except Exception:
            pass
        if "power_w" not in out:
            try:
                p = amdsmi.amdsmi_get_power_info(h)
                for key in ("current_socket_power", "socket_power", "average_socket_power"):
                    v = _num(p.get(key))
                    if v:
                        out["power_w"] = v
                        break
            except Exception:
                pass
        if "sclk_mhz" not in out:
            try:
                c = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)
                for key in ("clk", "cur_clk"):
                    v = _num(c.get(key))
                    if v:
                        out["sclk_mhz"] = v
                        break
            except Exception:
                pass
        return out

    if not read():
        return None
    return read


class Sampler:
    """Samples shader clock and board power every ``period`` seconds between start() and stop()."""

    def __init__(self, device: int = 0, period: float = 0.01):
        self.period = period
        bdf = pci_bus_id(device)
        self.bdf = bdf
        self.source = None
        self._read = None
        for name, make in (("amdsmi", _amdsmi_reader), ("sysfs_hwmon", _sysfs_reader)):
            r = make(bdf)
            if r is not None:
                self.source, self._read = name, r
                break
        self.samples: List[Dict[str, float]] = []
        self._stop = threading.Event()
        self._thread = None

    def _loop(self):
        while not self._stop.is_set():
            s = self._read()
            if s:
                self.samples.append(s)
            time.sleep(self.period)

    def start(self):
        self.samples = []
        if self._read is None:
            return self
        self._stop.clear()
        self._thread = threading.Thread(target=self._loop, daemon=True)
        self._thread.start()
        return self

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
            self._thread = None
        return self.summary()

    def summary(self) -> Dict[str, object]:
        """Median / min / max over the samples taken while the GPU was busy:
        graphics activity >= 90% where the source reports it, or >= 50% when
        fewer than 5 samples reach 90% (steps of many short kernels, whose
        launch gaps lower the averaged activity figure)."""
        busy, thr = [], 90.0
        for thr in (90.0, 50.0):
            busy = [s for s in self.samples if s.get("activity_pct", 100.0) >= thr]
            if len(busy) >= 5:
                break
        out: Dict[str, object] = {"source": self.source, "pci_bus_id": self.bdf, "samples": len(self.samples),
                                  "busy_samples": len(busy), "busy_threshold_pct": thr}
        act = [s["activity_pct"] for s in self.samples if "activity_pct" in s]
        if act:
            out["activity_pct_median"] = round(statistics.median(act), 1)
        else:  # no activity figure: every sample counts
            out["busy_threshold_pct"] = None
        for key, name in (("sclk_mhz", "sclk_mhz"), ("power_w", "power_w")):
            v = [s[key] for s in busy if key in s]
            if v:
                out[name] = {"median": round(statistics.median(v), 1), "min": round(min(v), 1),
                             "max": round(max(v), 1)}
        return out


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo ('' if unknown)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


if __name__ == "__main__":
    s = Sampler()
    s.start()
    time.sleep(0.2)
    print(s.stop())
    print("cpu:", cpu_model(), "affinity cores:", len(os.sched_getaffinity(0)))
